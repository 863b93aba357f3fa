"""Host check of the arithmetic identity the quantization kernels rely on.

The kernels never divide per element: they form the correctly rounded quotient
RN((x - mn) / s) from a correctly rounded reciprocal and one FMA correction step
(Markstein's theorem).  tests/c/quotient_check.c compares that construction with
IEEE division over every positive float16 scale, densely around every code boundary
and tie.  The GPU parity tests then check the kernels' codes bit for bit against
the oracle, which divides.
"""
import os
import shutil
import subprocess

import pytest

from tests.conftest import ROOT


def test_fma_corrected_quotient_equals_ieee_division(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler on this host")
    src = os.path.join(ROOT, "tests", "c", "quotient_check.c")
    exe = str(tmp_path / "quotient_check")
    subprocess.run([cc, "-O2", "-ffp-contract=off", src, "-o", exe, "-lm"], check=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout
    assert "0 mismatches" in out.stdout
