"""Pins for the oracle's Adam step, overflow check and loss-scale policy.

Every pin compares the oracle with something other than itself:

* first step from m = v = 0: the bias corrections make m^ = g and v^ = g^2,
  so the update is exactly -lr * g / (|g| + eps) (checked per element, with
  gradients both far above eps and comparable to it);
* k steps of one constant gradient: m^ = g and v^ = g^2 at every step, so
  p_k = p_0 - k * lr * g / (|g| + eps);
* g = 0: only the decoupled decay acts;
* beta1 = beta2 = 0: the moments forget their history;
* the pages' lost update: master 1.0 moves by ~1e-4 but the FP16 copy stays 1.0;
* loss scaling by a power of two and then undoing it changes nothing;
* the concatenation of N shard updates equals the unsharded update;
* an FP64 evaluation of the same update bounds the FP32 rounding error;
* the flag of the overflow check against positions of planted inf/NaN, and
  its sum of squares against an exactly rounded sum (math.fsum);
* the skip policy: an overflowing step leaves every array untouched, keeps t
  and halves S.
"""
import math
import os

import numpy as np
import pytest

import oracle

U32 = 2.0 ** -24  # unit roundoff of binary32


def ulp32(x):
    x = np.abs(np.asarray(x, np.float32))
    return (np.nextafter(x, np.float32(np.inf)) - x).astype(np.float64)


def f16_bits(x):
    return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def make_state(n, seed, g_std=1e-3, p_std=0.02, dtype="f16"):
    rng = np.random.default_rng(seed)
    g = rng.standard_normal(n).astype(np.float32) * np.float32(g_std)
    if dtype == "f16":
        g16 = g.astype(np.float16).view(np.uint16)
    else:
        g16 = oracle.encode16(g, "bf16")  # any bf16 pattern will do as input
    master = (rng.standard_normal(n) * p_std).astype(np.float32)
    return g16, master, np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)


HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)


@pytest.mark.parametrize("loss_scale,dtype", [(1.0, "f16"), (65536.0, "f16"), (1.0, "bf16"),
                                              (1024.0, "bf16")])
def test_first_step_closed_form(loss_scale, dtype):
    n = 20000
    g16, master, m, v, w16 = make_state(n, 11, dtype=dtype)
    p0 = master.astype(np.float64).copy()
    oracle.adam_step(w16, g16, master, m, v, dtype, step=1, loss_scale=loss_scale, **HP)
    g = oracle.decode16(g16, dtype).astype(np.float64) / loss_scale  # exact: S is a power of 2
    lr, eps = float(np.float32(HP["lr"])), float(np.float32(HP["eps"]))
    exact = p0 - lr * g / (np.abs(g) + eps)
    err = np.abs(master.astype(np.float64) - exact)
    # about 8 roundings on the update term, one on the final subtraction
    bound = 12 * U32 * lr + ulp32(np.maximum(np.abs(p0), lr))
    assert np.all(err <= bound), float(np.max(err / bound))
    # moments after one step: m = (1-b1) g, v = (1-b2) g^2, one or two roundings
    assert np.allclose(m, (1 - np.float32(0.9)) * g, rtol=2 * U32, atol=0)
    assert np.allclose(v, (1 - np.float32(0.999)) * g * g, rtol=3 * U32, atol=1e-45)
    # when |g| is comparable with eps, eps visibly shrinks the step
    if loss_scale == 65536.0:
        frac = np.abs(p0 - master.astype(np.float64)) / lr
        assert frac.min() < 0.5 and frac.max() < 1.0


def test_constant_gradient_closed_form():
    n, k = 5000, 10
    g16, master, m, v, w16 = make_state(n, 12)
    p0 = master.astype(np.float64).copy()
    for t in range(1, k + 1):
        oracle.adam_step(w16, g16, master, m, v, "f16", step=t, loss_scale=1.0, **HP)
    g = oracle.decode16(g16, "f16").astype(np.float64)
    lr = float(np.float32(HP["lr"]))
    exact = p0 - k * lr * g / (np.abs(g) + float(np.float32(1e-8)))
    err = np.abs(master.astype(np.float64) - exact)
    # step t's update term carries ~(10 + 3t) roundings of |lr|; each step adds
    # half an ulp of |p| from the subtraction.
    bound = sum((10 + 3 * t) for t in range(1, k + 1)) * U32 * lr + \
        k * ulp32(np.maximum(np.abs(p0), k * lr))
    assert np.all(err <= bound), float(np.max(err / bound))


@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_zero_gradient_only_decay_acts(wd):
    n = 4096
    _, master, m, v, w16 = make_state(n, 13)
    g16 = np.zeros(n, np.uint16)
    p0 = master.copy()
    for t in (1, 2, 3):
        oracle.adam_step(w16, g16, master, m, v, "f16", step=t, loss_scale=1.0,
                         lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=wd)
    assert not m.any() and not v.any()
    expect = p0.astype(np.float64) * (1 - float(np.float32(1e-3)) * float(np.float32(wd))) ** 3
    err = np.abs(master.astype(np.float64) - expect)
    if wd == 0.0:
        assert np.array_equal(master, p0)
    else:
        assert np.all(err <= 3 * ulp32(p0))
        assert np.all(np.abs(master) < np.abs(p0)) or not p0.any()


def test_zero_betas_forget_history():
    n = 4096
    g16, master, m, v, w16 = make_state(n, 14)
    rng = np.random.default_rng(99)
    m[:] = rng.standard_normal(n).astype(np.float32)
    v[:] = rng.random(n).astype(np.float32)
    p0 = master.astype(np.float64).copy()
    oracle.adam_step(w16, g16, master, m, v, "f16", step=7, loss_scale=1.0,
                     lr=1e-3, beta1=0.0, beta2=0.0, eps=1e-8, weight_decay=0.0)
    g = oracle.decode16(g16, "f16").astype(np.float64)
    assert np.array_equal(m.astype(np.float64), g)
    assert np.allclose(v.astype(np.float64), g * g, rtol=U32, atol=0)
    exact = p0 - float(np.float32(1e-3)) * g / (np.abs(g) + float(np.float32(1e-8)))
    assert np.all(np.abs(master - exact) <= 8 * U32 * 1e-3 + ulp32(np.maximum(np.abs(p0), 1e-3)))


def test_lost_update_in_fp16_working_copy(golden_dir):
    # master 1.0, lr 1e-4, first step: the master copy moves by about 1e-4,
    # the FP16 working copy cannot (the gap after 1.0 is 2^-10).
    with open(os.path.join(golden_dir, "lost_update.tsv")) as f:
        w, upd, _, result = [l for l in f if not l.startswith("#")][0].split("\t")
    master = np.array([float(w)], np.float32)
    g16 = f16_bits([-1e-3])
    m = np.zeros(1, np.float32)
    v = np.zeros(1, np.float32)
    w16 = np.zeros(1, np.uint16)
    oracle.adam_step(w16, g16, master, m, v, "f16", step=1, loss_scale=1.0,
                     lr=float(upd), beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)
    assert abs(float(master[0]) - (float(w) + float(upd))) < 1e-7
    assert master[0] > 1.0
    assert oracle.decode16(w16, "f16")[0] == float(result)


@pytest.mark.parametrize("k", [1, 4, 10])
def test_loss_scale_power_of_two_is_transparent(k):
    n = 8192
    rng = np.random.default_rng(15)
    # FP16 gradients in the normal range whose 2^k multiple is still exact
    g = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    g = np.clip(g, -1.0, 1.0)
    g = np.where(np.abs(g) < 1e-3, np.float32(1e-3), g)
    g16 = g.astype(np.float16).view(np.uint16)
    scaled = (g16.view(np.float16).astype(np.float32) * np.float32(2.0 ** k)).astype(np.float16)
    assert np.array_equal(scaled.astype(np.float32) / np.float32(2.0 ** k),
                          g16.view(np.float16).astype(np.float32))
    a = make_state(n, 16)
    b = [x.copy() for x in a]
    for t in (1, 2):
        oracle.adam_step(a[4], g16, a[1], a[2], a[3], "f16", step=t, loss_scale=1.0, **HP)
        oracle.adam_step(b[4], scaled.view(np.uint16), b[1], b[2], b[3], "f16", step=t,
                         loss_scale=2.0 ** k, **HP)
    for x, y in zip(a[1:], b[1:]):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("psi,n", [(10_000, 8), (10_007, 8), (999, 64), (50, 8)])
def test_shards_concatenate_to_unsharded_update(psi, n):
    g16, master, m, v, w16 = make_state(psi, 17)
    full = [x.copy() for x in (w16, master, m, v)]
    hp = dict(HP, weight_decay=0.01)
    for t in (1, 2, 3):
        oracle.adam_step(full[0], g16, full[1], full[2], full[3], "f16", step=t,
                         loss_scale=1024.0, **hp)
    parts = [x.copy() for x in (w16, master, m, v)]
    covered = 0
    for r in range(n):
        lay = oracle.layout(psi, n, r)
        sl = slice(lay.offset, lay.offset + lay.count)
        views = [np.ascontiguousarray(x[sl]) for x in parts]
        gv = np.ascontiguousarray(g16[sl])
        for t in (1, 2, 3):
            oracle.adam_step(views[0], gv, views[1], views[2], views[3], "f16", step=t,
                             loss_scale=1024.0, **hp)
        for x, y in zip(parts, views):
            x[sl] = y
        covered += lay.count
    assert covered == psi
    for x, y in zip(full, parts):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("dtype,wd", [("f16", 0.0), ("bf16", 0.01)])
def test_fp32_oracle_within_rounding_of_fp64(dtype, wd):
    n = 50000
    g16, master, m, v, w16 = make_state(n, 18, dtype=dtype)
    M, Mm, Mv = master.astype(np.float64), m.astype(np.float64), v.astype(np.float64)
    hp = dict(HP, weight_decay=wd)
    for t in (1, 2, 3):
        oracle.adam_step(w16, g16, master, m, v, dtype, step=t, loss_scale=1.0, **hp)
        oracle.adam_step_f64(M, Mm, Mv, g16, dtype, step=t, loss_scale=1.0, **hp)
    # three steps: each update term of size <= lr carries ~20 roundings, each
    # subtraction half an ulp of |p|
    bound = 3 * 20 * U32 * 1e-3 + 3 * ulp32(np.abs(M))
    assert np.all(np.abs(master - M) <= bound), float(np.max(np.abs(master - M) / bound))
    assert np.max(np.abs(m - Mm) / np.maximum(np.abs(Mm), 1e-30)) <= 40 * U32 or \
        np.max(np.abs(m - Mm)) <= 1e-12
    assert np.max(np.abs(v - Mv) / np.maximum(np.abs(Mv), 1e-38)) <= 16 * U32
    # the working copy is the master copy rounded to the 16-bit format
    assert np.array_equal(w16, oracle.encode16(master, dtype))


def test_overflow_flag_positions():
    n = 10000
    g16 = f16_bits(np.random.default_rng(19).standard_normal(n) * 1e-3)
    assert oracle.overflow_check(g16, "f16", 1.0)[0] == 0
    for pos in (0, 1, 7, 8, n // 2, n - 8, n - 1):
        for bad in (0x7C00, 0xFC00, 0x7E00, 0xFE01):
            h = g16.copy()
            h[pos] = bad
            assert oracle.overflow_check(h, "f16", 1.0)[0] == 1
            # the same inf/NaN outside the range handed over is not seen
            assert oracle.overflow_check(np.ascontiguousarray(np.delete(h, pos)), "f16",
                                         1.0)[0] == 0


def test_overflow_after_unscaling():
    # finite 16-bit values can still overflow FP32 once divided by a tiny S
    g16 = f16_bits([60000.0, 1.0])
    assert oracle.overflow_check(g16, "f16", 1.0)[0] == 0
    assert oracle.overflow_check(g16, "f16", 1e-35)[0] == 1
    bf = oracle.encode16(np.array([3e38, -1.0], np.float32), "bf16")
    assert oracle.overflow_check(bf, "bf16", 1.0)[0] == 0
    assert oracle.overflow_check(bf, "bf16", 0.5)[0] == 1


@pytest.mark.parametrize("dtype,S", [("f16", 1.0), ("f16", 65536.0), ("bf16", 1.0), ("f16", 3.0)])
def test_sum_of_squares_is_fsum(dtype, S):
    n = 30000
    rng = np.random.default_rng(20)
    x = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    g16 = x.astype(np.float16).view(np.uint16) if dtype == "f16" else oracle.encode16(x, dtype)
    flag, s = oracle.overflow_check(g16, dtype, S)
    g = oracle.decode16(g16, dtype) / np.float32(S)  # FP32 division, as the step does
    exact = math.fsum(float(a) * float(a) for a in g)
    assert flag == 0
    assert abs(s - exact) <= n * 2.0 ** -53 * exact


def test_skip_policy_trace():
    # overflow on every even step out of 10, starting from S = 65536
    st = oracle.ScalerState(loss_scale=65536.0)
    applied = []
    for step in range(1, 11):
        found = 1 if step % 2 == 0 else 0
        if oracle.policy(st, found):
            applied.append(st.step)
    assert applied == [1, 2, 3, 4, 5]
    assert st.step == 5
    assert st.loss_scale == 65536.0 / 2 ** 5 == 2048.0


def test_growth_after_clean_run():
    st = oracle.ScalerState(loss_scale=1024.0, growth_interval=3)
    used = []
    for _ in range(3):
        used.append(st.loss_scale)
        assert oracle.policy(st, 0)
    assert used == [1024.0] * 3       # the third update still unscales by 1024
    assert st.loss_scale == 2048.0 and st.step == 3
    assert not oracle.policy(st, 1)
    assert st.loss_scale == 1024.0 and st.step == 3


def test_skipped_step_touches_nothing():
    # the host never calls the step on overflow: after (clean, overflow) the
    # arrays equal those after the clean step alone, t is 1 and S has halved
    n = 2048
    a = make_state(n, 21)
    b = [x.copy() for x in a]
    st_a, st_b = oracle.ScalerState(65536.0), oracle.ScalerState(65536.0)
    for found in (0, 1):
        S = st_a.loss_scale
        if oracle.policy(st_a, found):
            oracle.adam_step(a[4], a[0], a[1], a[2], a[3], "f16", step=st_a.step,
                             loss_scale=S, **HP)
    S = st_b.loss_scale
    if oracle.policy(st_b, 0):
        oracle.adam_step(b[4], b[0], b[1], b[2], b[3], "f16", step=st_b.step,
                         loss_scale=S, **HP)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    assert st_a.step == st_b.step == 1
    assert st_a.loss_scale == 32768.0
