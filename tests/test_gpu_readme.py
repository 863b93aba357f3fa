"""The quick-start example in README.md runs as written and its output matches the
oracle on the same cache contents (so the example and the documented call sequence
stay correct)."""
import os
import re

import numpy as np
import pytest

import oracle as O
from tests.conftest import ROOT

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def test_readme_quick_start_runs_and_matches_the_oracle():
    text = open(os.path.join(ROOT, "README.md")).read()
    blocks = re.findall(r"```python\n(.*?)```", text, flags=re.S)
    assert len(blocks) == 1, "one python block in the README"
    print("[readme] quick start", flush=True)
    torch.manual_seed(0)
    ns = {}
    exec(compile(blocks[0], "README.md", "exec"), ns)
    K, V, q, out, dims, T0 = ns["K"], ns["V"], ns["q"], ns["out"], ns["dims"], ns["T0"]
    oc = O.LayerCache(dims.batch, dims.kv_heads, dims.head_dim, dims.bits, dims.group_k,
                      dims.group_v, dims.residual, dims.max_tokens)
    oc.prefill(K.cpu().numpy(), V.cpu().numpy())
    ref = oc.attend(q.cpu().numpy(), dims.head_dim ** -0.5)
    got = out.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= 2e-3 + 1e-3 * np.abs(ref))
