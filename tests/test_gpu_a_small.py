"""GPU parity, element by element, on small shards (seconds of oracle time).

Sizes span the kernels' head / 16-B tile / ragged tail split at every
alignment phase, both 16-bit formats, views of mismatched phase (the
element-wise kernel), the overflow flag at every kind of position, NaN
sentinels around the views (never read), the sum of squares, flag-gated
skipping, empty ranks and a non-default stream.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import zero_sharded_mixed_shard_amd as zs
from gpu_util import (GuardedView, assert_close, f32, line_head, log, u16)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
TD = {"f16": torch.float16, "bf16": torch.bfloat16}


def run_case(count, dtype, phases, steps=3, S=1.0, hp=HP, seed=1, grad_std=1e-3, psi=None,
             n=1, rank=0):
    psi = count if psi is None else psi
    td = TD[dtype]
    V = {k: GuardedView(count, td if k in ("g16", "w16") else torch.float32, phases[k], DEV)
         for k in ("g16", "w16", "master", "m", "v")}
    master0 = synth.fill_normal_(torch.empty(count), 0.02, seed)
    V["master"].view.copy_(master0.to(DEV))
    for k in ("m", "v", "w16"):
        V[k].view.zero_()
    host = dict(master=master0.numpy().copy(), m=np.zeros(count, np.float32),
                v=np.zeros(count, np.float32), w16=np.zeros(count, np.uint16))
    for t in range(1, steps + 1):
        g = synth.fill_normal_(torch.empty(count, dtype=td), grad_std, seed * 100 + t)
        V["g16"].view.copy_(g.to(DEV))
        zs.zero_adam_step(V["w16"].view, V["g16"].view, V["master"].view, V["m"].view,
                          V["v"].view, psi, n, rank, step=t, loss_scale=S, **hp)
        oracle.adam_step(host["w16"], u16(g), host["master"], host["m"], host["v"], dtype,
                         step=t, loss_scale=S, **hp)
    torch.cuda.synchronize()
    gpu = dict(master=f32(V["master"].view), m=f32(V["m"].view), v=f32(V["v"].view),
               w16=u16(V["w16"].view))
    stats = assert_close(gpu, host, dtype, f"count={count} phases={phases}")
    for k, gv in V.items():
        assert gv.guards_intact(), (k, count, phases)
    return stats


COUNTS = [1, 2, 3, 4, 5, 7, 8, 9, 63, 64, 65, 255, 256, 257, 1023, 1024, 1025, 2047, 2048, 2049,
          2050, 4095, 4096, 4097, 6161, 65541, 614431]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("phase", [0, 1, 2, 3])
def test_step_sizes_at_each_phase(dtype, phase):
    log(f"step sizes dtype={dtype} phase={phase}")
    worst = {}
    for count in COUNTS:
        st = run_case(count, dtype, dict.fromkeys(("g16", "w16", "master", "m", "v"), phase))
        for k, (mx, nz) in st.items():
            worst[k] = max(worst.get(k, 0), mx)
    log("  max ulp", worst)


@pytest.mark.parametrize("phases", [
    dict(g16=1, w16=0, master=0, m=0, v=0),
    dict(g16=0, w16=3, master=0, m=0, v=0),
    dict(g16=0, w16=0, master=0, m=2, v=0),
    dict(g16=2, w16=1, master=3, m=1, v=2),
])
def test_step_mismatched_phases_use_the_elementwise_kernel(phases):
    log(f"mismatched phases {phases}")
    for count in (1, 5, 1000, 4097, 65541):
        for dtype in ("f16", "bf16"):
            run_case(count, dtype, phases)


@pytest.mark.parametrize("S", [1.0, 3.0, 1024.0, 65536.0, 0.25])
def test_step_loss_scales(S):
    log(f"loss scale {S}")
    run_case(9000, "f16", dict.fromkeys(("g16", "w16", "master", "m", "v"), 0), S=S)
    run_case(9000, "bf16", dict.fromkeys(("g16", "w16", "master", "m", "v"), 1), S=S)


def test_step_hyperparameter_corners():
    ph = dict.fromkeys(("g16", "w16", "master", "m", "v"), 0)
    for hp in (dict(lr=1e-3, beta1=0.0, beta2=0.0, eps=1e-8, weight_decay=0.0),
               dict(lr=0.0, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1),
               dict(lr=1e-2, beta1=0.5, beta2=0.9, eps=0.0, weight_decay=0.0),
               dict(lr=-1e-3, beta1=0.99, beta2=0.9999, eps=1e-6, weight_decay=1.0)):
        log(f"hp {hp}")
        run_case(5003, "f16", ph, hp=hp, steps=4)


def test_step_subnormal_gradients_survive():
    # N(0, 1e-6) FP16 gradients are mostly FP16 subnormals
    ph = dict.fromkeys(("g16", "w16", "master", "m", "v"), 0)
    run_case(50000, "f16", ph, grad_std=1e-6)
    run_case(50000, "bf16", ph, grad_std=1e-30)


def test_step_ragged_rank_of_a_sharded_buffer():
    # psi = 10,007 over 8 ranks: ranks 0..6 own 1,251, rank 7 owns 1,250
    for r in (0, 6, 7):
        lay = oracle.layout(10_007, 8, r)
        run_case(lay.count, "f16", dict.fromkeys(("g16", "w16", "master", "m", "v"), 0),
                 psi=10_007, n=8, rank=r)


def test_step_empty_rank_touches_nothing():
    # psi = 10 over 8 ranks: rank 7 owns nothing
    lay = zs.zero_shard_layout(10, 8, 7)
    assert lay.count == 0
    views = [GuardedView(0, torch.float16, 0, DEV), GuardedView(0, torch.float16, 0, DEV)] + \
        [GuardedView(0, torch.float32, 0, DEV) for _ in range(3)]
    zs.zero_adam_step(*(v.view for v in views), 10, 8, 7, step=1, loss_scale=1.0, **HP)
    torch.cuda.synchronize()
    assert all(v.guards_intact() for v in views)


def test_step_skipped_on_device_when_flag_is_set():
    count = 70001
    td = torch.float16
    g = synth.fill_normal_(torch.empty(count, dtype=td), 1e-3, 5).to(DEV)
    master = synth.fill_normal_(torch.empty(count), 0.02, 6).to(DEV)
    m = torch.full((count,), 0.5, device=DEV)
    v = torch.full((count,), 0.25, device=DEV)
    w = torch.zeros(count, dtype=td, device=DEV)
    before = [x.clone() for x in (w, master, m, v)]
    flag = torch.ones(1, dtype=torch.int32, device=DEV)
    zs.zero_adam_step(w, g, master, m, v, count, 1, 0, step=3, loss_scale=1.0, found_inf=flag,
                      **HP)
    torch.cuda.synchronize()
    for a, b in zip((w, master, m, v), before):
        assert torch.equal(a.view(torch.int16) if a.dtype == td else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == td else b.view(torch.int32))
    flag.zero_()
    zs.zero_adam_step(w, g, master, m, v, count, 1, 0, step=3, loss_scale=1.0, found_inf=flag,
                      **HP)
    torch.cuda.synchronize()
    host = [u16(before[0]), u16(g), f32(before[1]), f32(before[2]), f32(before[3])]
    oracle.adam_step(host[0], host[1], host[2], host[3], host[4], "f16", step=3, loss_scale=1.0,
                     **HP)
    assert_close(dict(w16=u16(w), master=f32(master), m=f32(m), v=f32(v)),
                 dict(w16=host[0], master=host[2], m=host[3], v=host[4]), "f16")


def test_step_on_a_side_stream():
    count = 123457
    s = torch.cuda.Stream(device=DEV)
    g = synth.fill_normal_(torch.empty(count, dtype=torch.bfloat16), 1e-4, 7)
    master0 = synth.fill_normal_(torch.empty(count), 0.02, 8)
    with torch.cuda.stream(s):
        dg, dmaster = g.to(DEV), master0.to(DEV)
        dm = torch.zeros(count, device=DEV)
        dv = torch.zeros(count, device=DEV)
        dw = torch.zeros(count, dtype=torch.bfloat16, device=DEV)
        zs.zero_adam_step(dw, dg, dmaster, dm, dv, count, 1, 0, step=1, loss_scale=1.0, **HP)
    s.synchronize()
    host = dict(w16=np.zeros(count, np.uint16), master=master0.numpy().copy(),
                m=np.zeros(count, np.float32), v=np.zeros(count, np.float32))
    oracle.adam_step(host["w16"], u16(g), host["master"], host["m"], host["v"], "bf16", step=1,
                     loss_scale=1.0, **HP)
    assert_close(dict(w16=u16(dw), master=f32(dmaster), m=f32(dm), v=f32(dv)), host, "bf16")


def test_binding_rejects_short_tensors():
    t16 = torch.zeros(10, dtype=torch.float16, device=DEV)
    t32 = torch.zeros(10, device=DEV)
    with pytest.raises(ValueError):
        zs.zero_adam_step(t16, t16, t32, t32, t32, 11, 1, 0, step=1, loss_scale=1.0, **HP)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        zs.zero_overflow_check(t16, 11, 1, 0, 1.0, flag)
    with pytest.raises(zs.ZeroError):
        zs.zero_adam_step(t16, t16, t32, t32, t32, 10, 1, 0, step=0, loss_scale=1.0, **HP)


# ---- overflow check -----------------------------------------------------------

BAD = {"f16": (0x7C00, 0xFC00, 0x7E00), "bf16": (0x7F80, 0xFF80, 0x7FC0)}


def check_case(bits: np.ndarray, dtype, phase, S, sumsq=True):
    count = bits.size
    gv = GuardedView(count, TD[dtype], phase, DEV)  # guards hold NaN sentinels
    gv.view.copy_(torch.from_numpy(bits.view(np.int16).copy()).view(TD[dtype]).to(DEV))
    flag = torch.full((1,), 7, dtype=torch.int32, device=DEV)
    s = torch.full((1,), -1.0, device=DEV) if sumsq else None
    parts = torch.empty(zs.SUMSQ_PARTIALS, dtype=torch.float64, device=DEV) if sumsq else None
    zs.zero_overflow_check(gv.view, count, 1, 0, S, flag, s, parts)
    torch.cuda.synchronize()
    ref_flag, ref_s = oracle.overflow_check(bits, dtype, S)
    assert int(flag.item()) == ref_flag, (count, phase, S)
    if sumsq and ref_flag == 0:
        with np.errstate(over="ignore"):  # a sum past the FP32 range rounds to inf on both sides
            want = np.float32(ref_s)
        assert oracle.ulp_distance32(np.float32(s.item()), want).max() <= 1, (s.item(), ref_s)
    assert gv.guards_intact()
    return int(flag.item()), (s.item() if sumsq else None)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_overflow_flag_positions_and_phases(dtype):
    rng = np.random.default_rng(3)
    for count in (1, 7, 8, 9, 17, 4096 * 8 + 3, 300001):
        x = (rng.standard_normal(count) * 1e-3).astype(np.float32)
        bits = oracle.encode16(x, dtype)
        for phase in (0, 1, 2, 3, 5, 7, 39, 40):
            assert check_case(bits, dtype, phase, 1.0)[0] == 0
            head = line_head(phase, 2)   # first element of the vector part
            cand = {0, head, head - 1, head + 1, count // 2, count - 1, count - 8}
            for pos in sorted(p for p in cand if 0 <= p < count):
                for bad in BAD[dtype]:
                    b = bits.copy()
                    b[pos] = bad
                    assert check_case(b, dtype, phase, 1.0, sumsq=False)[0] == 1


def test_overflow_after_unscaling_on_device():
    bits = oracle.encode16(np.array([60000.0, 1.0, -2.0] * 1000, np.float32), "f16")
    assert check_case(bits, "f16", 0, 1.0)[0] == 0
    assert check_case(bits, "f16", 0, 1e-35)[0] == 1
    bf = oracle.encode16(np.array([3e38, -1.0] * 777, np.float32), "bf16")
    assert check_case(bf, "bf16", 3, 1.0)[0] == 0
    assert check_case(bf, "bf16", 3, 0.5)[0] == 1


def test_overflow_sumsq_large_grid_and_repeatable():
    rng = np.random.default_rng(4)
    count = 40_000_003          # enough vectors to cap the grid and loop in it
    x = (rng.standard_normal(count) * 1e-3).astype(np.float32)
    bits = x.astype(np.float16).view(np.uint16)
    f1, s1 = check_case(bits, "f16", 5, 1024.0)
    f2, s2 = check_case(bits, "f16", 5, 1024.0)
    assert f1 == f2 == 0 and s1 == s2
    b = bits.copy()
    b[rng.integers(0, count, 3)] = 0x7E00
    assert check_case(b, "f16", 5, 1024.0, sumsq=False)[0] == 1


def test_overflow_check_of_empty_rank_clears_outputs():
    flag = torch.full((1,), 7, dtype=torch.int32, device=DEV)
    s = torch.full((1,), 3.0, device=DEV)
    parts = torch.empty(zs.SUMSQ_PARTIALS, dtype=torch.float64, device=DEV)
    empty = torch.empty(0, dtype=torch.float16, device=DEV)
    zs.zero_overflow_check(empty, 10, 8, 6, 1.0, flag, s, parts)
    torch.cuda.synchronize()
    assert flag.item() == 0 and s.item() == 0.0


def test_short_names_match_the_entry_points():
    # adam_step(betas=...) and overflow_check(sumsq=...) without partials are the
    # same calls as zero_adam_step / zero_overflow_check
    count, psi, n, rank = 70_001, 560_008, 8, 7
    g = synth.fill_normal_(torch.empty(count, dtype=torch.float16), 1e-3, 61).to(DEV)
    master0 = synth.fill_normal_(torch.empty(count), 0.02, 62).to(DEV)
    A = dict(master=master0.clone(), m=torch.zeros(count, device=DEV),
             v=torch.zeros(count, device=DEV), w16=torch.zeros(count, dtype=torch.float16, device=DEV))
    B = {k: t.clone() for k, t in A.items()}
    for t in (1, 2):
        zs.adam_step(A["w16"], g, A["master"], A["m"], A["v"], psi, n, rank, lr=1e-3,
                     betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01, step=t, loss_scale=4.0)
        zs.zero_adam_step(B["w16"], g, B["master"], B["m"], B["v"], psi, n, rank, lr=1e-3,
                          beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=t,
                          loss_scale=4.0)
    torch.cuda.synchronize()
    for k in A:
        assert torch.equal(A[k].view(torch.int16 if A[k].dtype == torch.float16 else torch.int32),
                           B[k].view(torch.int16 if B[k].dtype == torch.float16 else torch.int32)), k
    f1 = torch.zeros(1, dtype=torch.int32, device=DEV)
    f2 = torch.zeros(1, dtype=torch.int32, device=DEV)
    s1, s2 = torch.zeros(1, device=DEV), torch.zeros(1, device=DEV)
    parts = torch.empty(zs.SUMSQ_PARTIALS, dtype=torch.float64, device=DEV)
    zs.overflow_check(g, psi, n, rank, 4.0, f1, sumsq=s1)
    zs.zero_overflow_check(g, psi, n, rank, 4.0, f2, s2, parts)
    torch.cuda.synchronize()
    assert f1.item() == f2.item() == 0 and s1.item() == s2.item() > 0


def test_sumsq_power_of_two_scales_and_their_edges():
    # S a power of two with a normal reciprocal takes the multiply path; the
    # others (non-powers, subnormal S, reciprocal below the normal range)
    # divide.  Flag and sum of squares agree with the oracle on both sides.
    rng = np.random.default_rng(8)
    count = 50_021
    x = (rng.standard_normal(count) * 1e-3).astype(np.float32)
    x[::97] *= 1e-4                      # some gradients deep in the FP16 subnormal range
    for dtype in ("f16", "bf16"):
        bits = oracle.encode16(x, dtype)
        for S in (2.0 ** -149, 2.0 ** -127, 2.0 ** -126, 2.0 ** -125, 0.75, 1.0, 3.0, 1024.0,
                  65536.0, float(np.nextafter(np.float32(65536.0), np.float32(0))),
                  2.0 ** 126, 2.0 ** 127):
            for phase in (0, 3):
                check_case(bits, dtype, phase, S)    # flag bit-exact; sum within 1 ulp


def test_sumsq_single_quotients_bit_exact():
    # One gradient per call: the sum of squares is then q*q rounded once to
    # FP32, so a single quotient q = g / S off by one unit would show.  Every
    # S path (power of two: multiply; others: the FP64 reciprocal product, and
    # the division where the quotient is subnormal) against the oracle's
    # correctly rounded FP32 division, bit for bit.
    rng = np.random.default_rng(11)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    s = torch.zeros(1, device=DEV)
    parts = torch.empty(zs.SUMSQ_PARTIALS, dtype=torch.float64, device=DEV)
    scales = [3.0, 7.0, 1000.0, 0.3, 1.0 + 2.0 ** -23, 2.0 - 2.0 ** -23, 65535.0, 2.0 ** 20 * 3.0,
              float(np.float32(1e30)), float(np.float32(3e-30)), 1024.0, 0.5]
    scales += [float(v) for v in (np.exp(rng.uniform(-40, 40, 24))).astype(np.float32)]
    n = 0
    for dtype, td in (("f16", torch.float16), ("bf16", torch.bfloat16)):
        pats = rng.integers(0, 1 << 16, 48).astype(np.uint16)
        pats[:4] = [0x0001, 0x8003, 0x03ff, 0x3c01]       # subnormals and 1 + 1 ulp (FP16 bits)
        for h in pats:
            bits = np.array([h], np.uint16)
            g = torch.from_numpy(bits.view(np.int16).copy()).view(td).to(DEV)
            for S in scales:
                zs.zero_overflow_check(g, 1, 1, 0, S, flag, s, parts)
                rf, rs = oracle.overflow_check(bits, dtype, S)
                got_f, got_s = int(flag.item()), s.item()
                assert got_f == rf, (dtype, hex(int(h)), S)
                if rf == 0:
                    with np.errstate(over="ignore"):
                        want = np.float32(rs)
                    assert np.float32(got_s).view(np.uint32) == want.view(np.uint32), \
                        (dtype, hex(int(h)), S, got_s, rs)
                n += 1
    log(f"single-gradient sums of squares: {n} cases bit-exact")


def test_sumsq_quotients_inside_vectors_bit_exact():
    # Quotients at every place a gradient can sit (head, each lane of a 16-B
    # vector, the vectors in flight and the remainder, the tail) in shards of
    # zeros, for scales that are not powers of two: a quotient below the
    # normal range (divided), one near 2^-125 (either side of the test), and
    # a normal quotient in a vector whose zeros send it down the per-element
    # branch (the product kept).  With at most two nonzero squares every
    # summation order gives the same FP64 value, so the FP64 partial sums
    # (the kernel's scratch, zero-filled first; white-box) must add up to the
    # oracle's FP64 sum bit for bit, and the FP32 result must match too.
    rng = np.random.default_rng(12)
    scales = [3.0, 1000.0, float(np.float32(0.3)), 6.0, 3.0 * 2.0 ** 20, 3.0 * 2.0 ** 100]
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    s = torch.zeros(1, device=DEV)
    parts = torch.zeros(zs.SUMSQ_PARTIALS, dtype=torch.float64, device=DEV)
    count = 20_011
    n_cases = n_divided = 0

    def encode(x, fmt):
        x = np.array([x], np.float32)
        b = int(x.view(np.uint32)[0]) if fmt == "f32" else int(oracle.encode16(x, fmt)[0])
        return b if b & 0x7fffffff else 1            # never zero: the smallest subnormal

    def value(b, fmt):
        if fmt == "f32":
            return float(np.uint32(b).view(np.float32))
        return float(oracle.decode16(np.array([b], np.uint16), fmt)[0])

    for fmt in ("f16", "bf16", "f32"):
        for phase in (0, 5):
            gv = GuardedView(count, torch.float32 if fmt == "f32" else TD[fmt], phase, DEV)
            head = line_head(phase, 4 if fmt == "f32" else 2)
            per_vec = 4 if fmt == "f32" else 8
            pos = sorted({*range(0, min(head, 3)), head - 1, *range(head, head + per_vec + 1),
                          count // 2, count // 2 + 1, count - 9, count - 2, count - 1,
                          *rng.integers(head, count, 6).tolist()} - {-1})
            for S in scales:
                for p in pos:
                    q = p + 1 if p + 1 < count else p - 1
                    sign = 1.0 if rng.random() < 0.5 else -1.0
                    tiny = encode(sign * S * 2.0 ** rng.uniform(-152, -124), fmt)
                    normal = encode(2.0 ** rng.uniform(-10, 10), fmt)
                    for placed in (((p, tiny),), ((p, tiny), (q, normal)), ((p, normal),)):
                        bits = np.zeros(count, np.uint32 if fmt == "f32" else np.uint16)
                        for i, b in placed:
                            bits[i] = b
                        parts.zero_()
                        if fmt == "f32":
                            gv.view.copy_(torch.from_numpy(bits.view(np.float32)).to(DEV))
                            zs.zero_overflow_check_g32(gv.view, count, 1, 0, S, flag, s, parts)
                            rf, rs = oracle.overflow_check_g32(bits.view(np.float32), S)
                        else:
                            gv.view.copy_(torch.from_numpy(bits.view(np.int16).copy())
                                          .view(TD[fmt]).to(DEV))
                            zs.zero_overflow_check(gv.view, count, 1, 0, S, flag, s, parts)
                            rf, rs = oracle.overflow_check(bits, fmt, S)
                        got = parts.cpu().numpy().sum()
                        case = (fmt, phase, S, [(i, hex(b)) for i, b in placed])
                        assert int(flag.item()) == rf == 0, case
                        assert np.float64(got).view(np.uint64) == np.float64(rs).view(np.uint64), \
                            (case, got, rs)
                        assert np.float32(s.item()).view(np.uint32) == \
                            np.float32(rs).view(np.uint32), case
                        n_cases += 1
                        n_divided += any(abs(value(b, fmt) / S) < 2.0 ** -126 for _, b in placed)
            assert gv.guards_intact()
    log(f"sums of squares with quotients inside vectors: {n_cases} cases bit-exact "
        f"({n_divided} with a subnormal quotient)")


def test_calls_return_without_synchronising():
    # A bounded spin kernel ahead of them on the stream: the check and the step
    # are enqueued behind it and the calls return while it still runs.
    count = 50_000
    g = synth.fill_normal_(torch.empty(count, dtype=torch.float16), 1e-3, 71).to(DEV)
    master = synth.fill_normal_(torch.empty(count), 0.02, 72).to(DEV)
    m = torch.zeros(count, device=DEV)
    v = torch.zeros(count, device=DEV)
    w = torch.zeros(count, dtype=torch.float16, device=DEV)
    flag = torch.full((1,), 5, dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()
    torch.cuda._sleep(50_000_000)             # bounded spin: tens of ms at shader clocks
    zs.zero_overflow_check(g, count, 1, 0, 1.0, flag)
    zs.zero_adam_step(w, g, master, m, v, count, 1, 0, step=1, loss_scale=1.0, found_inf=flag,
                      **HP)
    done = torch.cuda.Event()
    done.record()
    pending = not done.query()
    torch.cuda.synchronize()
    assert pending, "a call waited for the stream"
    h_master = synth.fill_normal_(torch.empty(count), 0.02, 72).numpy().copy()
    h_m, h_v, h_w = np.zeros(count, np.float32), np.zeros(count, np.float32), np.zeros(count, np.uint16)
    oracle.adam_step(h_w, u16(g), h_master, h_m, h_v, "f16", step=1, loss_scale=1.0, **HP)
    assert flag.item() == 0
    assert_close(dict(master=f32(master), m=f32(m), v=f32(v), w16=u16(w)),
                 dict(master=h_master, m=h_m, v=h_v, w16=h_w), "f16", "async")


def test_concurrent_host_threads_on_their_own_streams():
    # The library keeps no per-call state; four host threads step four shards
    # on four streams at once and each result equals its sequential twin.
    import threading
    count, steps, nthreads = 120_001, 4, 4
    grads = [[synth.fill_normal_(torch.empty(count, dtype=torch.float16), 1e-3, 900 + 10 * k + t)
              .to(DEV) for t in range(steps)] for k in range(nthreads)]
    master0 = [synth.fill_normal_(torch.empty(count), 0.02, 950 + k).to(DEV) for k in range(nthreads)]

    def fresh(k):
        return dict(master=master0[k].clone(), m=torch.zeros(count, device=DEV),
                    v=torch.zeros(count, device=DEV),
                    w16=torch.zeros(count, dtype=torch.float16, device=DEV),
                    flag=torch.zeros(1, dtype=torch.int32, device=DEV))

    def run(k, st, stream, errors):
        try:
            with torch.cuda.stream(stream):
                for t in range(steps):
                    zs.zero_overflow_check(grads[k][t], count, 1, 0, 1024.0, st["flag"],
                                           stream=stream)
                    zs.zero_adam_step(st["w16"], grads[k][t], st["master"], st["m"], st["v"],
                                      count, 1, 0, step=t + 1, loss_scale=1024.0,
                                      found_inf=st["flag"], stream=stream, **HP)
        except Exception as e:          # noqa: BLE001  (reported below)
            errors.append(e)

    torch.cuda.synchronize()
    par = [fresh(k) for k in range(nthreads)]
    streams = [torch.cuda.Stream() for _ in range(nthreads)]
    errors = []
    threads = [threading.Thread(target=run, args=(k, par[k], streams[k], errors))
               for k in range(nthreads)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for k in range(nthreads):
        seq = fresh(k)
        run(k, seq, torch.cuda.current_stream(), errors)
        torch.cuda.synchronize()
        for key in ("master", "m", "v"):
            assert torch.equal(par[k][key].view(torch.int32), seq[key].view(torch.int32)), (k, key)
        assert torch.equal(par[k]["w16"].view(torch.int16), seq["w16"].view(torch.int16)), k
    assert not errors, errors
