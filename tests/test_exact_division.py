"""The reference mean divides a sum of at most 8 FP8 e4m3fn values by k = 1..8. The
kernels replace the IEEE division by q = s * RN(1/k) plus one fused residual
correction; this test checks, exhaustively over every such sum and k, that the result
is the correctly rounded quotient (C, correctly rounded fmaf)."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_small_divisor_division_is_correctly_rounded(tmp_path):
    exe = tmp_path / "exact_div_check"
    src = os.path.join(HERE, "support", "exact_div_check.c")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", src, "-o", str(exe), "-lm"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout
    assert "mismatches 0" in r.stdout
