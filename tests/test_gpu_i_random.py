"""Seeded random parity sweep: check -> decision -> step against the oracle.

Each case draws the elements per launch (half the cases the library's rule,
the others random pieces of whole tiles), a shard size (1 to ~300k elements,
biased toward tile and line boundaries), view phases (all equal, or mixed:
the element-wise kernel),
a 16-bit format, hyperparameters (including beta = 0, eps = 0, wd = 0 and
negative lr), a loss scale (powers of two and not), a gradient spread from
deep in the FP16 subnormal range to values that overflow after unscaling,
and sometimes planted inf/NaN.  The flag, the skip-or-apply decision and
the state after up to three steps must meet the parity bar.  Further sweeps
cover the FP32-gradient path, the reduce-scatter and all-gather stand-ins
(random rank counts, formats, phases, shards in place) and device-controlled
schedules.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import zero_sharded_mixed_shard_amd as zs
from gpu_util import GuardedView, assert_close, f32, log, u16

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TD = {"f16": torch.float16, "bf16": torch.bfloat16}
KEYS = ("g16", "w16", "master", "m", "v")
N_CASES = 400


def draw_case(rng):
    base = int(rng.choice([1, 7, 64, 1024, 2048, 4096, 65536, 262144]))
    count = max(1, base + int(rng.integers(-40, 41)) if rng.random() < 0.7
                else int(rng.integers(1, 300_000)))
    if rng.random() < 0.75:
        p = int(rng.integers(0, 40))
        phases = dict.fromkeys(KEYS, p)
    else:
        phases = {k: int(rng.integers(0, 8)) for k in KEYS}
    dtype = "f16" if rng.random() < 0.5 else "bf16"
    hp = dict(lr=float(rng.choice([0.0, 1e-4, 1e-3, 3e-3, -1e-3])),
              beta1=float(rng.choice([0.0, 0.5, 0.9])),
              beta2=float(rng.choice([0.0, 0.99, 0.999, 0.9999])),
              eps=float(rng.choice([0.0, 1e-8, 1e-6])),
              weight_decay=float(rng.choice([0.0, 0.01, 0.1])))
    S = float(rng.choice([1.0, 1024.0, 65536.0, 3.0, 0.5, 2.0 ** -20, 1000.0]))
    std = float(10.0 ** rng.uniform(-7, 4.5))
    inject = rng.random() < 0.15
    steps = int(rng.integers(1, 4))
    return count, phases, dtype, hp, S, std, inject, steps


def draw_piece(prng, count):
    """Elements per launch for one case, from a generator of its own (so the cases
    themselves are the same with or without it): half the cases the library's
    rule, the others pieces of 1 to ~count/2048 tiles plus a remainder."""
    if prng.random() < 0.5:
        return 0
    return int(prng.integers(1, count // 2048 + 2)) * 2048 + int(prng.integers(0, 2048))


@pytest.fixture
def launch_pieces():
    yield
    torch.cuda.synchronize()
    zs.zero_set_launch_piece(0)


def test_random_sweep_matches_oracle(launch_pieces):
    rng = np.random.default_rng(20261202)
    prng = np.random.default_rng(31)
    stats = {"cases": 0, "skipped_steps": 0, "applied_steps": 0, "mixed_phase": 0, "split": 0}
    worst = {k: [0, 0] for k in ("master", "m", "v", "w16")}   # max ulp, non-bitwise count
    for case in range(N_CASES):
        count, phases, dtype, hp, S, std, inject, steps = draw_case(rng)
        piece = draw_piece(prng, count)
        zs.zero_set_launch_piece(piece)
        # split for sure: more whole tiles than a piece holds, whatever the head
        stats["split"] += piece != 0 and max(0, count - 63) // 2048 > piece // 2048
        td = TD[dtype]
        V = {k: GuardedView(count, td if k in ("g16", "w16") else torch.float32, phases[k], DEV)
             for k in KEYS}
        master0 = synth.fill_normal_(torch.empty(count), 0.02, 7000 + case)
        V["master"].view.copy_(master0.to(DEV))
        for k in ("m", "v", "w16"):
            V[k].view.zero_()
        ref = dict(master=master0.numpy().copy(), m=np.zeros(count, np.float32),
                   v=np.zeros(count, np.float32), w16=np.zeros(count, np.uint16))
        flag = torch.zeros(1, dtype=torch.int32, device=DEV)
        t = 0
        for s in range(steps):
            g = synth.fill_normal_(torch.empty(count, dtype=td), std, 8000 + 10 * case + s)
            if inject:
                synth.inject_nonfinite_(g, min(1.0, 2.0 / count), 9000 + 10 * case + s)
            gh = u16(g)
            V["g16"].view.copy_(g.to(DEV))
            zs.zero_overflow_check(V["g16"].view, count, 1, 0, S, flag)
            ref_flag, _ = oracle.overflow_check(gh, dtype, S)
            got_flag = int(flag.item())
            assert got_flag == ref_flag, (case, s, count, phases, dtype, S, std)
            if got_flag:
                stats["skipped_steps"] += 1
                continue
            t += 1
            stats["applied_steps"] += 1
            zs.zero_adam_step(V["w16"].view, V["g16"].view, V["master"].view, V["m"].view,
                              V["v"].view, count, 1, 0, step=t, loss_scale=S, found_inf=flag,
                              **hp)
            oracle.adam_step(ref["w16"], gh, ref["master"], ref["m"], ref["v"], dtype, step=t,
                             loss_scale=S, **hp)
        torch.cuda.synchronize()
        got = dict(master=f32(V["master"].view), m=f32(V["m"].view), v=f32(V["v"].view),
                   w16=u16(V["w16"].view))
        st = assert_close(got, ref, dtype, f"case {case}: count={count} phases={phases} {dtype} "
                                           f"hp={hp} S={S} std={std:.3g} piece={piece}")
        for k, (mx, nz) in st.items():
            worst[k][0] = max(worst[k][0], mx)
            worst[k][1] += nz
        assert all(x.guards_intact() for x in V.values()), case
        stats["cases"] += 1
        stats["mixed_phase"] += len(set(phases.values())) > 1
    log(f"random sweep: {stats}; max ulp / non-bitwise elements {worst}")
    assert stats["skipped_steps"] > 0 and stats["applied_steps"] > 0 and stats["mixed_phase"] > 0
    assert stats["split"] > 0


def test_random_fp32_gradients_device_control_and_exchanges(launch_pieces):
    rng = np.random.default_rng(4242)
    prng = np.random.default_rng(32)
    for case in range(120):
        count = int(rng.choice([1, 5, 1023, 2049, 4096 + 31, 70_001, 200_003]))
        piece = draw_piece(prng, count)
        zs.zero_set_launch_piece(piece)
        dtype = "f16" if case % 2 else "bf16"
        pa, pg = int(rng.integers(0, 8)), int(rng.integers(0, 8))
        S = float(rng.choice([1.0, 256.0, 3.0, 65536.0]))
        std = float(10.0 ** rng.uniform(-6, 1))
        hp = dict(lr=float(rng.choice([1e-4, 1e-3])), beta1=0.9, beta2=0.999,
                  eps=float(rng.choice([0.0, 1e-8])), weight_decay=float(rng.choice([0.0, 0.01])))
        # micro-batches into an FP32 accumulator, the FP32 check with its sum of squares
        acc = GuardedView(count, torch.float32, pa, DEV)
        gv = GuardedView(count, TD[dtype], pg, DEV)
        ref_acc = np.zeros(count, np.float32)
        for j in range(int(rng.integers(1, 4))):
            g = synth.fill_normal_(torch.empty(count, dtype=TD[dtype]), std, 20_000 + 10 * case + j)
            gv.view.copy_(g.to(DEV))
            zs.zero_grad_accumulate(acc.view, gv.view, count, 1, 0, first=(j == 0))
            oracle.grad_accumulate(ref_acc, u16(g), dtype, first=(j == 0))
        torch.cuda.synchronize()
        assert np.array_equal(f32(acc.view).view(np.uint32), ref_acc.view(np.uint32)), (case, piece)
        flag = torch.zeros(1, dtype=torch.int32, device=DEV)
        ssq = torch.zeros(1, device=DEV)
        parts = torch.empty(zs.SUMSQ_PARTIALS, dtype=torch.float64, device=DEV)
        zs.zero_overflow_check_g32(acc.view, count, 1, 0, S, flag, ssq, parts)
        rf, rs = oracle.overflow_check_g32(ref_acc, S)
        assert int(flag.item()) == rf, case
        if rf == 0:
            assert oracle.ulp_distance32(np.float32(ssq.item()), np.float32(rs)).max() <= 1, case
            V = {k: GuardedView(count, torch.float32, pa, DEV) for k in ("master", "m", "v")}
            V["w16"] = GuardedView(count, TD[dtype], pa, DEV)
            master0 = synth.fill_normal_(torch.empty(count), 0.02, 21_000 + case)
            V["master"].view.copy_(master0.to(DEV))
            for k in ("m", "v", "w16"):
                V[k].view.zero_()
            zs.zero_adam_step_g32(V["w16"].view, acc.view, V["master"].view, V["m"].view,
                                  V["v"].view, count, 1, 0, step=1, loss_scale=S, **hp)
            ref = dict(master=master0.numpy().copy(), m=np.zeros(count, np.float32),
                       v=np.zeros(count, np.float32), w16=np.zeros(count, np.uint16))
            oracle.adam_step_g32(ref["w16"], ref_acc, ref["master"], ref["m"], ref["v"], dtype,
                                 step=1, loss_scale=S, **hp)
            torch.cuda.synchronize()
            got = dict(master=f32(V["master"].view), m=f32(V["m"].view), v=f32(V["v"].view),
                       w16=u16(V["w16"].view))
            assert_close(got, ref, dtype, f"g32 case {case} piece {piece}")
        # the exchanges over a random rank count and formats
        psi = int(rng.integers(1, 150_000))
        n = int(rng.integers(1, 17))
        fin, fout = rng.choice(["f16", "bf16", "f32"], 2)
        tdi = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}
        reps = []
        for k in range(n):
            x = synth.fill_normal_(torch.empty(psi, dtype=tdi[fin]), 1e-2, 30_000 + 100 * case + k)
            reps.append(x.to(DEV))
        hreps = [f32(r) if fin == "f32" else u16(r) for r in reps]
        rank = int(rng.integers(0, n))
        lay = zs.zero_shard_layout(psi, n, rank)
        out = GuardedView(lay.count, tdi[fout], int(rng.integers(0, 8)), DEV)
        zs.zero_reduce_shard(out.view, reps, psi, n, rank)
        want = oracle.reduce_shard(hreps, fin, fout, psi, n, rank)
        got = f32(out.view) if fout == "f32" else u16(out.view)
        assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), (case, psi, n, fin, fout)
        assert out.guards_intact()
    log("random FP32-gradient and exchange sweep: 120 cases")


def test_random_gathers():
    # random rank counts, formats and phases; some shards already in place in the
    # full buffer; the padded tail and every guard must come back untouched
    rng = np.random.default_rng(9090)
    tdi = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}
    host = lambda t, fmt: f32(t) if fmt == "f32" else u16(t)
    in_place = 0
    for case in range(80):
        psi = int(rng.integers(1, 150_000))
        n = int(rng.integers(1, 17))
        fmt = str(rng.choice(["f16", "bf16", "f32"]))
        lays = [zs.zero_shard_layout(psi, n, k) for k in range(n)]
        total = lays[0].padded_total
        full = GuardedView(total, tdi[fmt], int(rng.integers(0, 8)), DEV)
        full.view.copy_(synth.fill_normal_(torch.empty(total, dtype=tdi[fmt]), 1.0,
                                           31_000 + case).to(DEV))
        shards, owners, hshards = [], [], []
        for k, lay in enumerate(lays):
            vals = synth.fill_normal_(torch.empty(lay.count, dtype=tdi[fmt]), 1e-2,
                                      32_000 + 100 * case + k)
            hshards.append(host(vals, fmt))
            if lay.count and rng.random() < 0.3:
                view = full.view[lay.offset:lay.offset + lay.count]
                in_place += 1
            else:
                owners.append(GuardedView(lay.count, tdi[fmt], int(rng.integers(0, 8)), DEV))
                view = owners[-1].view
            view.copy_(vals.to(DEV))
            shards.append(view)
        want = oracle.gather_shards(hshards, psi, n, host(full.view, fmt))
        zs.zero_gather_shards(full.view, shards, psi, n)
        got = host(full.view, fmt)
        assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), (case, psi, n, fmt)
        assert full.guards_intact() and all(o.guards_intact() for o in owners), case
    assert in_place > 0
    log(f"random gathers: 80 cases, {in_place} shards in place")


def test_random_device_control_schedules():
    # random overflow schedules and growth intervals, enqueued without read-back
    from test_gpu_c_device_ctl import make_grads, run_device, run_oracle
    rng = np.random.default_rng(777)
    for case in range(12):
        count = int(rng.choice([3, 4099, 65_537]))
        steps = int(rng.integers(2, 9))
        bad = tuple(int(s) for s in np.nonzero(rng.random(steps) < 0.3)[0] + 1)
        growth = int(rng.choice([1, 2, 3, 2000]))
        dtype = "f16" if case % 2 else "bf16"
        S0 = float(rng.choice([1.0, 1024.0, 65536.0]))
        grads = make_grads(count, steps, dtype, 600 + 50 * case, bad_steps=bad)
        got, ctl, master0 = run_device(count, dtype, grads, S0, growth, phase=case % 4)
        ref, st, trace = run_oracle(master0, grads, dtype, S0, growth)
        assert (ctl.scaler.step, ctl.scaler.loss_scale, ctl.scaler.clean_steps) == \
            (st.step, st.loss_scale, st.clean_steps), (case, trace)
        assert_close(got, ref, dtype, f"device-control case {case}: bad {bad} growth {growth}")
    log("random device-control schedules: 12 cases")
