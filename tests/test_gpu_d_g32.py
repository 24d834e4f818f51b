"""GPU parity of the FP32-gradient path: accumulation of 16-bit micro-batches
in FP32, the check over FP32 gradients and the step reading them, element by
element against the oracle, at every alignment phase and across tile and
ragged-tail sizes, plus a whole accumulate -> check -> step sequence.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import zero_sharded_mixed_shard_amd as zs
from gpu_util import GuardedView, assert_close, f32, line_head, log, u16

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TD = {"f16": torch.float16, "bf16": torch.bfloat16}
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
COUNTS = [1, 3, 4, 5, 1023, 2047, 2048, 2049, 4097, 65541, 300007]


def micro_batches(count, k, dtype, seed):
    return [synth.fill_normal_(torch.empty(count, dtype=TD[dtype]), 1e-3, seed + j)
            for j in range(k)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("phases", [(0, 0), (1, 1), (3, 3), (0, 1), (2, 0)])
def test_accumulate_matches_oracle(dtype, phases):
    pa, pg = phases
    for count in COUNTS:
        mbs = micro_batches(count, 4, dtype, 900)
        acc = GuardedView(count, torch.float32, pa, DEV)
        gv = GuardedView(count, TD[dtype], pg, DEV)
        ref = np.zeros(count, np.float32)
        for j, g in enumerate(mbs):
            gv.view.copy_(g.to(DEV))
            zs.zero_grad_accumulate(acc.view, gv.view, count, 1, 0, first=(j == 0))
            oracle.grad_accumulate(ref, u16(g), dtype, first=(j == 0))
        torch.cuda.synchronize()
        got = f32(acc.view)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (count, phases)
        assert acc.guards_intact() and gv.guards_intact()
    log(f"accumulate {dtype} phases {phases}: bitwise")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("phases", [(0, 0), (1, 1), (3, 3), (0, 1)])
def test_fused_accumulate_check_matches_oracle(dtype, phases):
    # the last micro-batch accumulated with the FP32 check of the result fused
    # in: the accumulator bit for bit and the flag equal to the check's flag on
    # the result -- clean, with an inf in the last micro-batch, with a NaN from
    # an earlier one, for S a power of two and not
    pa, pg = phases
    rng = np.random.default_rng(17 + pa + 4 * pg)
    for count in COUNTS:
        for case in ("clean", "inf_last", "nan_first"):
            for S in (1024.0, 3.0):
                mbs = micro_batches(count, 3, dtype, 950 + count % 97)
                pos = int(rng.integers(count))
                if case == "inf_last":
                    mbs[-1][pos] = float("-inf")
                elif case == "nan_first":
                    mbs[0][pos] = float("nan")
                acc = GuardedView(count, torch.float32, pa, DEV)
                gv = GuardedView(count, TD[dtype], pg, DEV)
                flag = torch.full((1,), 7, dtype=torch.int32, device=DEV)
                ref = np.zeros(count, np.float32)
                for j, g in enumerate(mbs):
                    gv.view.copy_(g.to(DEV))
                    if j == len(mbs) - 1:
                        zs.zero_grad_accumulate_check(acc.view, gv.view, count, 1, 0,
                                                      first=(j == 0), loss_scale=S,
                                                      found_inf=flag)
                    else:
                        zs.zero_grad_accumulate(acc.view, gv.view, count, 1, 0, first=(j == 0))
                    oracle.grad_accumulate(ref, u16(g), dtype, first=(j == 0))
                torch.cuda.synchronize()
                rf, _ = oracle.overflow_check_g32(ref, S)
                assert rf == (case != "clean")
                assert flag.item() == rf, (count, case, S, phases)
                got = f32(acc.view)
                same = (got.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(got) & np.isnan(ref))
                assert same.all(), (count, case, S, phases)
                assert acc.guards_intact() and gv.guards_intact()
    log(f"fused accumulate + check {dtype} phases {phases}: bitwise, flags equal")


def test_fused_accumulate_check_overflow_by_division_and_empty_rank():
    # BF16 gradients near the top of the FP32 range: the FP32 sum overflows in
    # one case and only the division by S < 1 overflows in the other
    count = 70_001
    big = torch.full((count,), 1.0, dtype=torch.bfloat16)
    big[12_345] = 1.7e38
    g = big.to(DEV)
    acc = torch.empty(count, device=DEV)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    for first, S, want in ((True, 1.0, 0), (True, 0.25, 1), (False, 1.0, 1)):
        zs.zero_grad_accumulate_check(acc, g, count, 1, 0, first=first, loss_scale=S,
                                      found_inf=flag)
        torch.cuda.synchronize()
        assert flag.item() == want, (first, S)
    # second pass (not first): 1.7e38 + 1.7e38 overflows FP32 to inf
    assert np.isinf(f32(acc)[12_345])
    # an empty rank still clears the flag
    flag.fill_(7)
    zs.zero_grad_accumulate_check(acc[:0], g[:0], 10, 8, 7, first=True, loss_scale=1.0,
                                  found_inf=flag)
    torch.cuda.synchronize()
    assert flag.item() == 0


@pytest.mark.parametrize("phase", [0, 1, 2, 3])
def test_check_g32_matches_oracle(phase):
    rng = np.random.default_rng(40 + phase)
    for count in (1, 3, 4, 5, 4099, 1_000_003):
        x = (rng.standard_normal(count) * 1e-2).astype(np.float32)
        gv = GuardedView(count, torch.float32, phase, DEV)
        flag = torch.zeros(1, dtype=torch.int32, device=DEV)
        s = torch.zeros(1, device=DEV)
        parts = torch.empty(zs.SUMSQ_PARTIALS, dtype=torch.float64, device=DEV)
        for S in (1.0, 3.0, 65536.0):
            gv.view.copy_(torch.from_numpy(x).to(DEV))
            zs.zero_overflow_check_g32(gv.view, count, 1, 0, S, flag, s, parts)
            rf, rs = oracle.overflow_check_g32(x, S)
            assert flag.item() == rf == 0
            assert oracle.ulp_distance32(np.float32(s.item()), np.float32(rs)).max() <= 1
        head = line_head(phase, 4)   # first element of the vector part
        for pos in sorted({p for p in (0, head - 1, head, count // 2, count - 1)
                           if 0 <= p < count}):
            for bad in (np.inf, -np.inf, np.nan):
                y = x.copy()
                y[pos] = bad
                gv.view.copy_(torch.from_numpy(y).to(DEV))
                zs.zero_overflow_check_g32(gv.view, count, 1, 0, 1.0, flag)
                assert flag.item() == oracle.overflow_check_g32(y, 1.0)[0] == 1, (count, pos)
        assert gv.guards_intact()
    big = torch.tensor([3e38, 1.0], device=DEV)
    zs.zero_overflow_check_g32(big, 2, 1, 0, 0.5, flag)
    assert flag.item() == 1


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("phases", [(0, 0), (2, 2), (0, 1)])
def test_step_g32_matches_oracle(dtype, phases):
    pf, pg = phases    # FP32 state phase, FP32 gradient phase
    rng = np.random.default_rng(50)
    for count in COUNTS:
        V = {k: GuardedView(count, torch.float32, pf, DEV) for k in ("master", "m", "v")}
        V["w16"] = GuardedView(count, TD[dtype], pf, DEV)
        G = GuardedView(count, torch.float32, pg, DEV)
        master0 = (rng.standard_normal(count) * 0.02).astype(np.float32)
        V["master"].view.copy_(torch.from_numpy(master0).to(DEV))
        for k in ("m", "v", "w16"):
            V[k].view.zero_()
        ref = dict(master=master0.copy(), m=np.zeros(count, np.float32),
                   v=np.zeros(count, np.float32), w16=np.zeros(count, np.uint16))
        for t in (1, 2, 3):
            g = (rng.standard_normal(count) * 1e-3 * 1024).astype(np.float32)
            G.view.copy_(torch.from_numpy(g).to(DEV))
            zs.zero_adam_step_g32(V["w16"].view, G.view, V["master"].view, V["m"].view,
                                  V["v"].view, count, 1, 0, step=t, loss_scale=1024.0, **HP)
            oracle.adam_step_g32(ref["w16"], g, ref["master"], ref["m"], ref["v"], dtype, step=t,
                                 loss_scale=1024.0, **HP)
        torch.cuda.synchronize()
        got = dict(master=f32(V["master"].view), m=f32(V["m"].view), v=f32(V["v"].view),
                   w16=u16(V["w16"].view))
        assert_close(got, ref, dtype, f"g32 count={count} phases={phases}")
        assert all(x.guards_intact() for x in list(V.values()) + [G])


def test_accumulate_check_step_sequence_gpt2_rank():
    # GPT-2-small-shaped flat buffer, rank 5 of 8: 4 micro-batches accumulated
    # in FP32, then check and step on the FP32 gradients; every element checked
    w = synth.WORKLOADS[2]
    lay = zs.zero_shard_layout(w.psi, w.n, 5)
    cnt = lay.count
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay)
    acc = torch.empty(cnt, device=DEV)
    master = synth.fill_normal_(torch.empty(cnt, device=DEV), 0.02, 2201)
    m = torch.zeros(cnt, device=DEV)
    v = torch.zeros(cnt, device=DEV)
    w16 = torch.zeros(cnt, dtype=torch.float16, device=DEV)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    ref = dict(master=f32(master), m=np.zeros(cnt, np.float32), v=np.zeros(cnt, np.float32),
               w16=np.zeros(cnt, np.uint16))
    racc = np.zeros(cnt, np.float32)
    g = torch.empty(cnt, dtype=torch.float16, device=DEV)
    for t in (1, 2):
        for j in range(4):
            synth.fill_normal_(g, w.grad_std, synth.seed_of(2, 1, 10 * t + j))
            zs.zero_grad_accumulate(acc, g, w.psi, w.n, 5, first=(j == 0))
            oracle.grad_accumulate(racc, u16(g), "f16", first=(j == 0))
        zs.zero_overflow_check_g32(acc, w.psi, w.n, 5, w.loss_scale, flag)
        assert flag.item() == oracle.overflow_check_g32(racc, w.loss_scale)[0] == 0
        zs.zero_adam_step_g32(w16, acc, master, m, v, w.psi, w.n, 5, step=t,
                              loss_scale=w.loss_scale, found_inf=flag, **hp)
        oracle.adam_step_g32(ref["w16"], racc, ref["master"], ref["m"], ref["v"], "f16", step=t,
                             loss_scale=w.loss_scale, **hp)
    torch.cuda.synchronize()
    assert np.array_equal(f32(acc).view(np.uint32), racc.view(np.uint32))
    got = dict(master=f32(master), m=f32(m), v=f32(v), w16=u16(w16))
    log("  accumulate->check->step", assert_close(got, ref, "f16", "sequence"))
