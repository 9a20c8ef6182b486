"""The quantization kernels' fast quotient gives the codes of the division.

For scales from 2^-80 up the HIP quantization (quantize_rowwise_fp8,
quantize_tensorwise_fp8 and the fused decode path) forms x / scale as a
product with the reciprocal plus one fma correction.  That value can differ
from the IEEE quotient in its last bit; ``tests/quotient_exhaustive.c``
enumerates every bf16 amax and every bf16 x with |x| <= amax in both FP8
formats (about 2.1e9 pairs) and checks, with the oracle's encoder, that the
FP8 codes never differ at those scales.  The first differences lie far below
the threshold (scales under 2^-100), so the margin is checked as well.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "tests", "quotient_exhaustive.c"), os.path.join(ROOT, "oracle", "sfr_oracle.c")]


def test_fma_quotient_codes_exhaustive(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not installed")
    exe = str(tmp_path / "quotient_exhaustive")
    r = subprocess.run(["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                        *SRC, "-o", exe, "-lm"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr
    rows = re.findall(r"fmt (\d) pairs (\d+) differing_from_2\^-80 (\d+) largest_differing_scale (\S+)", r.stdout)
    assert len(rows) == 2, r.stdout
    for fmt, pairs, bad, worst in rows:
        assert int(pairs) > 1_000_000_000, r.stdout
        assert int(bad) == 0, r.stdout
        assert float.fromhex(worst) < 2.0 ** -100, r.stdout
