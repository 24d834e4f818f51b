"""The sum-of-squares kernel's unscaling shortcut, checked on the CPU.

For a loss scale S that is not a power of two the kernel forms g / S as one
FP64 product with RN64(1/S) rounded once to FP32, and divides only where that
product is below 2^-125 in magnitude.  tests/method/quotient_check.c compares
the shortcut with the correctly rounded FP32 division for every FP16 and BF16
gradient pattern against 2000 scales, and for 5e7 random FP32 pairs.  (The
argument that makes it exact: the product is within 2^-52 of g / S, which is
never within 2^-49 of an FP32 rounding midpoint.)
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_fp64_reciprocal_quotient_equals_the_division(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    exe = tmp_path / "quotient_check"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                    os.path.join(HERE, "method", "quotient_check.c"), "-lm", "-o", str(exe)],
                   check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    tried = int(r.stdout.split()[1])
    assert tried > 2.5e8, r.stdout
