"""Pins for the oracle's FP32-gradient functions (accumulate, check, step).

* the FP32-gradient step reduces to the 16-bit step when the FP32 gradients are
  exactly the decoded 16-bit ones (bit for bit), and follows the first-step
  closed form for FP32 gradients that no 16-bit format holds;
* accumulation: the first micro-batch is copied exactly; k micro-batches stay
  within the recursive-summation bound of the exact sum (math.fsum); exact
  when every partial sum is representable; and the pages' point holds: a
  16-bit accumulator loses contributions that the FP32 one keeps;
* the FP32 check flags planted inf/NaN, overflow made by the division, and its
  sum of squares is the exactly rounded sum of the same squares.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle

U32 = 2.0 ** -24
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def ulp32(x):
    x = np.abs(np.asarray(x, np.float32))
    return (np.nextafter(x, np.float32(np.inf)) - x).astype(np.float64)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_g32_step_reduces_to_16bit_step(dtype):
    n = 20000
    rng = np.random.default_rng(30)
    x = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    g16 = oracle.encode16(x, dtype)
    g32 = oracle.decode16(g16, dtype)
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    a = [np.zeros(n, np.uint16), master.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)]
    b = [z.copy() for z in a]
    for t in (1, 2, 3):
        oracle.adam_step(a[0], g16, a[1], a[2], a[3], dtype, step=t, loss_scale=4.0, **HP)
        oracle.adam_step_g32(b[0], g32, b[1], b[2], b[3], dtype, step=t, loss_scale=4.0, **HP)
    for y, z in zip(a, b):
        assert np.array_equal(y, z)


@pytest.mark.parametrize("S", [1.0, 65536.0])
def test_g32_first_step_closed_form(S):
    n = 20000
    rng = np.random.default_rng(31)
    g32 = (rng.standard_normal(n) * 1e-3 * rng.random(n)).astype(np.float32)  # not 16-bit values
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    master = p0.copy()
    m, v, w = np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)
    hp = dict(HP, weight_decay=0.0)
    oracle.adam_step_g32(w, g32, master, m, v, "f16", step=1, loss_scale=S, **hp)
    g = g32.astype(np.float64) / S
    lr, eps = float(np.float32(1e-3)), float(np.float32(1e-8))
    exact = p0.astype(np.float64) - lr * g / (np.abs(g) + eps)
    bound = 12 * U32 * lr + ulp32(np.maximum(np.abs(p0), lr))
    assert np.all(np.abs(master - exact) <= bound)
    assert np.array_equal(w, oracle.encode16(master, "f16"))


def test_accumulate_first_copies_exactly():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    for dtype in ("f16", "bf16"):
        acc = np.full(bits.size, 7.0, np.float32)
        oracle.grad_accumulate(acc, bits, dtype, first=True)
        ref = oracle.decode16(bits, dtype)
        nan = np.isnan(ref)
        assert np.array_equal(acc[~nan].view(np.uint32), ref[~nan].view(np.uint32))
        assert np.all(np.isnan(acc[nan]))


def test_accumulate_within_summation_bound():
    n, k = 4000, 16
    rng = np.random.default_rng(32)
    mbs = [oracle.encode16((rng.standard_normal(n) * 1e-3).astype(np.float32), "bf16")
           for _ in range(k)]
    acc = np.zeros(n, np.float32)
    for j, g in enumerate(mbs):
        oracle.grad_accumulate(acc, g, "bf16", first=(j == 0))
    vals = np.stack([oracle.decode16(g, "bf16").astype(np.float64) for g in mbs])
    exact = np.array([math.fsum(col) for col in vals.T])
    bound = (k - 1) * U32 * np.abs(vals).sum(axis=0) * (1 + 1e-6)
    assert np.all(np.abs(acc - exact) <= bound + 1e-45)


def test_accumulate_exact_when_representable():
    # integers of a few bits: every partial sum is an exact FP32 number
    n, k = 1000, 9
    rng = np.random.default_rng(33)
    ints = rng.integers(-50, 51, size=(k, n)).astype(np.float32)
    acc = np.zeros(n, np.float32)
    for j in range(k):
        oracle.grad_accumulate(acc, oracle.encode16(ints[j], "f16"), "f16", first=(j == 0))
    assert np.array_equal(acc, ints.sum(axis=0))


def test_fp32_accumulator_keeps_what_16bit_loses():
    # 1.0 then 64 micro-batches of ~1e-3: each is below half the BF16 gap
    # after 1.0 (2^-8), so a BF16 accumulator never moves; FP32 gets ~1.064
    one = oracle.encode16(np.array([1.0], np.float32), "bf16")
    small = oracle.encode16(np.array([1e-3], np.float32), "bf16")
    acc32 = np.zeros(1, np.float32)
    oracle.grad_accumulate(acc32, one, "bf16", first=True)
    acc16 = one.copy()
    for _ in range(64):
        oracle.grad_accumulate(acc32, small, "bf16", first=False)
        s = oracle.decode16(acc16, "bf16") + oracle.decode16(small, "bf16")
        acc16 = oracle.encode16(s, "bf16")
    step = float(Fraction(float(oracle.decode16(small, "bf16")[0])))
    assert oracle.decode16(acc16, "bf16")[0] == 1.0
    assert abs(float(acc32[0]) - (1.0 + 64 * step)) < 1e-6


def test_check_g32_flag_and_sumsq():
    n = 5000
    rng = np.random.default_rng(34)
    g = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    flag, s = oracle.overflow_check_g32(g, 3.0)
    q = g / np.float32(3.0)
    assert flag == 0
    exact = math.fsum(float(a) * float(a) for a in q)
    assert abs(s - exact) <= n * 2.0 ** -53 * exact
    for pos in (0, 1, n // 3, n - 1):
        for bad in (np.inf, -np.inf, np.nan):
            h = g.copy()
            h[pos] = bad
            assert oracle.overflow_check_g32(h, 3.0)[0] == 1
    big = np.array([3e38, 1.0], np.float32)
    assert oracle.overflow_check_g32(big, 1.0)[0] == 0
    assert oracle.overflow_check_g32(big, 0.5)[0] == 1
