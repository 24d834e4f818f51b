"""The kernels' quotient rule, checked on the CPU.

For a divisor d that is the same for every element -- a loss scale S that is
not a power of two (the step and the sum-of-squares check), and the bias
corrections 1 - beta^t (the step) -- the kernels form a / d as one FP64
product with RN64(1/d) rounded once to FP32, and divide only where that
result is below 2^-125 in magnitude and a is not zero.
tests/method/quotient_check.c compares the rule with the correctly rounded
FP32 division for every FP16 and BF16 pattern against 2000 scales, 5e7 random
FP32 pairs, 5e7 random FP32 numerators against bias corrections, and 6e7
numerators built to put the quotient within an ulp of an FP32 rounding
boundary.  (The argument that makes it exact: the product is within 2^-52 of
a / d, which is never within 2^-49 of an FP32 rounding boundary.)
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
    words = r.stdout.split()
    tried = int(words[1])
    assert tried > 3.5e8, r.stdout
    # each part ran: 16-bit patterns, random pairs, bias corrections, boundary cases
    parts = [int(w.strip(",()")) for w in (words[7], words[9], words[11], words[13])]
    assert parts[0] > 2.5e8 and parts[1] > 4e7 and parts[2] > 4e7 and parts[3] > 4e7, r.stdout
