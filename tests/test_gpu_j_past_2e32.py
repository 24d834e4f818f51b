"""The FP32-gradient path, the sums of squares and the exchanges past 2^32
elements (64-bit element indexing), on views that start 5 elements into their
allocations (a head done one element at a time, then line-aligned vectors).

Elementwise results are checked against the oracle on windows: both ends,
random positions and the one straddling element 2^32.  The sums of squares
are checked against their exact value, for inputs whose unscaled squares and
every partial sum are exact in FP64, so one rounding to FP32 is all that
separates them.  The flag is checked with a non-finite value planted past
element 2^32.
"""
import gc

import numpy as np
import pytest
import torch

import oracle
import synth
import zero_sharded_mixed_shard_amd as zs
from gpu_util import assert_close, f32, log, u16

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
N = 2 ** 32 + 3001
PHASE = 5
FAR = 2 ** 32 + 17


@pytest.fixture(autouse=True)
def _device_memory():
    free, _ = torch.cuda.mem_get_info(DEV)
    if free < 100e9:
        pytest.skip(f"needs 100 GB of device memory, {free / 1e9:.0f} GB free")
    yield
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def windows(count, rng, n_random=8, width=4096):
    w = [(0, width), (count - width, count), (2 ** 32 - width // 2, 2 ** 32 + width // 2)]
    for s in rng.integers(0, count - width, n_random):
        w.append((int(s), int(s) + width))
    return sorted(w)


def take(t, wins, conv):
    return [conv(t[a:b]) for a, b in wins]


def empty(count, dtype):
    return torch.empty(PHASE + count, dtype=dtype, device=DEV)[PHASE:]


def test_fp32_gradient_path_past_2e32():
    dt, td = "bf16", torch.bfloat16
    wins = windows(N, np.random.default_rng(32))
    log(f"accumulating two micro-batches of {N} BF16 gradients")
    g16 = empty(N, td)
    acc = empty(N, torch.float32)
    ref_acc = [np.zeros(b - a, np.float32) for a, b in wins]
    for j in range(2):
        synth.fill_normal_(g16, 1e-3, 40_000 + j)
        zs.zero_grad_accumulate(acc, g16, N, 1, 0, first=(j == 0))
        for r, g in zip(ref_acc, take(g16, wins, u16)):
            oracle.grad_accumulate(r, g, dt, first=(j == 0))
    torch.cuda.synchronize()
    for (a, _), got, want in zip(wins, take(acc, wins, f32), ref_acc):
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), a
    del g16

    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    zs.zero_overflow_check_g32(acc, N, 1, 0, 1.0, flag)
    assert flag.item() == 0
    log("FP32-gradient steps")
    master = synth.fill_normal_(empty(N, torch.float32), 0.02, 40_100)
    m = empty(N, torch.float32).zero_()
    v = empty(N, torch.float32).zero_()
    w16 = empty(N, td).zero_()
    host = [dict(master=a, m=np.zeros(a.size, np.float32), v=np.zeros(a.size, np.float32),
                 w16=np.zeros(a.size, np.uint16)) for a in take(master, wins, f32)]
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    for t in (1, 2):
        zs.zero_adam_step_g32(w16, acc, master, m, v, N, 1, 0, step=t, loss_scale=1.0,
                              found_inf=flag, **hp)
        for h, g in zip(host, ref_acc):
            oracle.adam_step_g32(h["w16"], g, h["master"], h["m"], h["v"], dt, step=t,
                                 loss_scale=1.0, **hp)
    torch.cuda.synchronize()
    got = [dict(master=a, m=b, v=c, w16=d) for a, b, c, d in
           zip(take(master, wins, f32), take(m, wins, f32), take(v, wins, f32),
               take(w16, wins, u16))]
    cat = lambda lst, k: np.concatenate([x[k] for x in lst])
    keys = ("master", "m", "v", "w16")
    log("  windows", assert_close({k: cat(got, k) for k in keys},
                                  {k: cat(host, k) for k in keys}, dt, "g32 past 2^32"))


def test_sums_of_squares_and_flags_past_2e32():
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    s = torch.zeros(1, device=DEV)
    parts = torch.empty(zs.SUMSQ_PARTIALS, dtype=torch.float64, device=DEV)
    # every unscaled gradient is exactly 1/4 (S a power of two: the multiply
    # path; S = 3: the division path), so the exact sum is N/16
    g32 = empty(N, torch.float32)
    for val, S in ((0.5, 2.0), (0.75, 3.0)):
        g32.fill_(val)
        zs.zero_overflow_check_g32(g32, N, 1, 0, S, flag, s, parts)
        assert flag.item() == 0
        assert s.item() == float(np.float32(N / 16)), (val, S, s.item())
    g32[FAR] = float("inf")
    zs.zero_overflow_check_g32(g32, N, 1, 0, 2.0, flag, s, parts)
    assert flag.item() == 1
    zs.zero_overflow_check_g32(g32, N, 1, 0, 2.0, flag)
    assert flag.item() == 1
    del g32
    for td in (torch.float16, torch.bfloat16):
        g16 = empty(N, td)
        for val, S, q2 in ((1.0, 1.0, 1.0), (0.75, 3.0, 1 / 16)):
            g16.fill_(val)
            zs.zero_overflow_check(g16, N, 1, 0, S, flag, s, parts)
            assert flag.item() == 0
            assert s.item() == float(np.float32(N * q2)), (td, val, S, s.item())
        g16[FAR] = float("nan")
        zs.zero_overflow_check(g16, N, 1, 0, 1.0, flag, s, parts)
        assert flag.item() == 1
        zs.zero_overflow_check(g16, N, 1, 0, 1.0, flag)
        assert flag.item() == 1
        g16[FAR] = 1.0
        zs.zero_overflow_check(g16, N, 1, 0, 1.0, flag)
        assert flag.item() == 0
        del g16


def test_exchanges_past_2e32():
    psi, n = 2 * N, 2                 # S = N: rank 1 owns elements [N, 2N)
    log(f"reduce-scatter and all-gather of {psi} FP16 elements over 2 ranks")
    reps = [synth.fill_normal_(torch.empty(psi, dtype=torch.float16, device=DEV), 1e-2,
                               41_000 + k) for k in range(n)]
    out = empty(N, torch.float32)
    zs.zero_reduce_shard(out, reps, psi, n, 1)
    torch.cuda.synchronize()
    wins = windows(N, np.random.default_rng(33))
    for (a, b), got in zip(wins, take(out, wins, f32)):
        # the same window as rank 1's whole chunk of a 2-rank buffer of 2(b - a) elements
        rw = [np.concatenate([np.zeros(b - a, np.uint16), u16(r[N + a:N + b])]) for r in reps]
        want = oracle.reduce_shard(rw, "f16", "f32", 2 * (b - a), n, 1)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), a
    del out
    # shard 0 shares its destination's alignment (vector copy); shard 1, 5
    # elements into its allocation, does not (element copy)
    sh1 = empty(N, torch.float16)
    sh1.copy_(reps[1][N:])
    full = torch.empty(psi, dtype=torch.float16, device=DEV)
    zs.zero_gather_shards(full, [reps[0][:N], sh1], psi, n)
    torch.cuda.synchronize()
    for a, b in wins:
        assert np.array_equal(u16(full[a:b]), u16(reps[0][a:b])), a
        assert np.array_equal(u16(full[N + a:N + b]), u16(sh1[a:b])), a
