"""bench.py --timeline on the timeline build of the library (libkivi_timeline.so): the
per-workgroup stamps come back for every launch and are ordered as the kernel takes its
steps (start, blocks done, arrival counted; in the last arriver its own stores complete,
partial loads complete, merge done), and the shader clock read from them is plausible.

Runs in a process of its own: the binding picks its library at import."""
import json
import os
import subprocess
import sys

import pytest

from tests.conftest import ROOT

pytestmark = pytest.mark.gpu


def test_timeline_stamps_are_ordered():
    lib = os.path.join(ROOT, "bit_quantization_amd", "libkivi_timeline.so")
    if not os.path.exists(lib):
        pytest.fail("libkivi_timeline.so is not built")
    print("[timeline] bench.py --timeline --workload llama8b_32k --copies 2", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--timeline",
                        "--workload", "llama8b_32k", "--copies", "2"],
                       capture_output=True, text=True, timeout=110, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    res = json.loads([l for l in r.stdout.splitlines() if l.startswith("{")][-1])
    assert res["workgroups"] == 256 and res["n_split"] == 4
    for name in ("back_to_back", "paused_5ms", "back_to_back_2"):
        s = res["series"][name]
        assert len(s["span_us"]) == 64 and len(s["clock_mhz"]) == 64
        m = s["median"]
        assert 0 <= m["start_spread_us"] < m["blocks_done_first_us"]
        assert m["blocks_done_first_us"] <= m["blocks_done_median_us"] <= m["blocks_done_last_us"]
        assert m["arrival_median_us"] <= m["arrival_last_us"] <= m["merge_done_last_us"]
        assert m["blocks_done_last_us"] <= m["arrival_last_us"]
        phases = [m["merger_stores_us"], m["merger_loads_us"], m["merger_fold_us"]]
        assert all(p is not None and p >= 0 for p in phases)
        assert sum(phases) <= m["span_us"]
        assert 0 < m["workgroup_stream_median_us"] <= m["blocks_done_last_us"]
        assert 500 < m["clock_mhz"] < 3000
