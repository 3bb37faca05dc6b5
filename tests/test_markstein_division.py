"""The Q/K quantizers take the quotient x / s under an E4M3 block scale s from the
correctly rounded reciprocal by one residual step (Markstein's division), not by an
IEEE division.  tests/markstein_check.c compares the two on the host for every float
x of one binade and every positive E4M3 scale (power-of-two scaling of x carries the
result to every binade whose quotients stay normal), so the step is exact for any
float input, not only the bf16 elements the GPU tests enumerate: the pre-processing
quantizer feeds it centered or rotated float values."""
import pathlib
import shutil
import subprocess

import pytest

SRC = pathlib.Path(__file__).with_name("markstein_check.c")


def test_markstein_quotient_equals_ieee_division(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = tmp_path / "markstein_check"
    subprocess.run([gcc, "-O2", "-std=c99", "-ffp-contract=off", "-o", str(exe), str(SRC), "-lm"], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("0 of 1056964608 "), res.stdout
