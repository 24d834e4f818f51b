"""GPU parity of the reduce-scatter stand-in with the overflow check fused in.

zero_reduce_shard_check must write the chunk zero_reduce_shard writes (the
oracle's FP32 sum in rank order, rounded once), bit for bit, and raise the flag
exactly when the oracle's check of that written chunk does (16-bit output: the
check of 16-bit gradients; FP32 output: the check of FP32 gradients), for
every pair of formats, ragged sizes, misaligned and mismatched views, planted
inf and NaN at head, vector and tail positions, sums that overflow the output
format, quotients that overflow FP32, an empty rank (the flag is still
cleared), an in-place reduce, the tile loops of a lowered grid cap, the
device-resident form that reads S from the control block, and a ZeRO-2 rank's
whole device-resident step (this reduce, the decision, the step) captured in a
HIP graph and replayed.
"""
import numpy as np
import pytest
import torch

import oracle
import zero_sharded_mixed_shard_amd as zs
from gpu_util import GuardedView, log
from test_gpu_e_exchange import TD, host, make_replicas

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
PAIRS = [("f16", "f16"), ("f16", "f32"), ("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32"),
         ("f32", "f16"), ("f32", "bf16")]


def oracle_flag(chunk: np.ndarray, out_fmt: str, S: float) -> int:
    if out_fmt == "f32":
        return oracle.overflow_check_g32(chunk, S)[0]
    return oracle.overflow_check(chunk, out_fmt, S)[0]


def plant(reps, pos, value):
    for r in reps:
        r[pos] = value


def run_case(reps, in_fmt, out_fmt, psi, n, rank, S, out_phase, what):
    hreps = [host(r) for r in reps]
    lay = zs.zero_shard_layout(psi, n, rank)
    out = GuardedView(lay.count, TD[out_fmt], out_phase, DEV)
    flag = torch.full((1,), 7, dtype=torch.int32, device=DEV)
    zs.zero_reduce_shard_check(out.view, reps, psi, n, rank, S, flag)
    want = oracle.reduce_shard(hreps, in_fmt, out_fmt, psi, n, rank)
    got = host(out.view)
    assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), what
    want_flag = oracle_flag(want, out_fmt, S) if lay.count else 0
    assert int(flag.item()) == want_flag, (what, int(flag.item()), want_flag)
    assert out.guards_intact(), what
    return want_flag


@pytest.mark.parametrize("in_fmt,out_fmt", PAIRS)
def test_reduce_check_matches_reduce_then_check(in_fmt, out_fmt):
    raised = 0
    for psi, n in ((10, 8), (1000, 8), (100_003, 8), (65_537, 3)):
        for phase in (0, 1):
            rank = n // 2 if n > 1 else 0
            lay = zs.zero_shard_layout(psi, n, rank)
            base = make_replicas(psi, n, in_fmt, 41 * psi + n, phase)
            # ordinary data, S a power of two and not
            for S in (1.0, 1024.0, 3.0):
                raised += run_case(base, in_fmt, out_fmt, psi, n, rank, S, phase,
                                   (in_fmt, out_fmt, psi, n, phase, S))
            if lay.count == 0:
                continue
            # planted inf / NaN at the chunk's first, middle and last elements, one replica
            for rel in (0, lay.count // 2, lay.count - 1):
                for bad in (float("inf"), float("nan"), float("-inf")):
                    reps = [r.clone() for r in base]
                    reps[n - 1][lay.offset + rel] = bad
                    raised += run_case(reps, in_fmt, out_fmt, psi, n, rank, 1.0, phase,
                                       (in_fmt, out_fmt, psi, n, phase, rel, bad))
            # a sum that overflows the output format (FP16: n * 30000 > 65504 for n >= 3)
            reps = [r.clone() for r in base]
            plant(reps, lay.offset + lay.count // 3, 30000.0 if in_fmt != "f32" else 3.0e38)
            raised += run_case(reps, in_fmt, out_fmt, psi, n, rank, 1.0, phase,
                               (in_fmt, out_fmt, psi, n, phase, "sum overflow"))
            # a quotient that overflows FP32: one finite sum near 60000 divided by a tiny S
            reps = [r.clone() for r in base]
            reps[0][lay.offset + (2 * lay.count) // 3] = 60000.0
            flagged = run_case(reps, in_fmt, out_fmt, psi, n, rank, 1e-35, phase,
                               (in_fmt, out_fmt, psi, n, phase, "quotient overflow"))
            assert flagged == 1
            raised += flagged
    assert raised > 0
    log(f"reduce+check {in_fmt}->{out_fmt}: bitwise chunks, flags equal ({raised} raised)")


def test_reduce_check_empty_rank_in_place_and_mismatched_views():
    # an empty rank still clears the flag
    reps = make_replicas(10, 8, "f16", 5)
    flag = torch.full((1,), 7, dtype=torch.int32, device=DEV)
    zs.zero_reduce_shard_check(torch.empty(0, dtype=torch.float16, device=DEV), reps, 10, 8, 7,
                               1.0, flag)
    assert int(flag.item()) == 0
    # in place: the output is exactly replica 0's chunk, with an inf planted in replica 2
    psi, n, rank = 40_003, 4, 2
    reps = make_replicas(psi, n, "bf16", 9)
    lay = zs.zero_shard_layout(psi, n, rank)
    reps[2][lay.offset + 17] = float("inf")
    hreps = [host(r) for r in reps]
    want = oracle.reduce_shard(hreps, "bf16", "bf16", psi, n, rank)
    zs.zero_reduce_shard_check(reps[0][lay.offset:lay.offset + lay.count], reps, psi, n, rank,
                               2.0, flag)
    assert np.array_equal(host(reps[0][lay.offset:lay.offset + lay.count]), want)
    assert int(flag.item()) == oracle_flag(want, "bf16", 2.0) == 1
    # replicas and output of different 16-B phases: the element-wise path
    reps = make_replicas(70_001, 3, "f16", 13, phase=1)
    reps[1][70_000] = float("nan")
    for out_phase in (0, 2, 3):
        run_case(reps, "f16", "f16", 70_001, 3, 2, 1.0, out_phase, ("mismatched", out_phase))
        run_case(reps, "f16", "f32", 70_001, 3, 0, 1.0, out_phase, ("mismatched f32", out_phase))
    log("reduce+check: empty rank clears the flag; in place; element-wise path")


def test_reduce_check_tile_loops():
    # a grid cap of 3 blocks: every block walks many tiles, then raises its flag
    zs.zero_set_grid_cap(3)
    try:
        for in_fmt, out_fmt in (("f16", "f16"), ("f32", "bf16")):
            psi, n = 200_003, 4
            base = make_replicas(psi, n, in_fmt, 77)
            for rank in (0, 3):
                lay = zs.zero_shard_layout(psi, n, rank)
                run_case(base, in_fmt, out_fmt, psi, n, rank, 1.0, 0, ("cap", rank))
                reps = [r.clone() for r in base]
                reps[0][lay.offset + lay.count - 1] = float("inf")
                assert run_case(reps, in_fmt, out_fmt, psi, n, rank, 1.0, 0, ("cap inf", rank))
    finally:
        torch.cuda.synchronize()
        zs.zero_set_grid_cap(0)
    log("reduce+check under a grid cap of 3 blocks: bitwise, flags equal")


def test_reduce_check_device_control():
    # S from the control block, the flag into it; the decision that follows skips
    psi, n, rank = 300_001, 8, 5
    reps = make_replicas(psi, n, "f16", 23)
    lay = zs.zero_shard_layout(psi, n, rank)
    hreps = [host(r) for r in reps]
    want = oracle.reduce_shard(hreps, "f16", "f16", psi, n, rank)
    for S in (65536.0, 3.0, 1e-37):
        ctl = zs.device_ctl_new(S, DEV)
        out = GuardedView(lay.count, torch.float16, 1, DEV)
        zs.zero_reduce_shard_check_dev(out.view, reps, psi, n, rank, ctl)
        c = zs.device_ctl_read(ctl)
        assert np.array_equal(host(out.view), want)
        assert c.found_inf == oracle_flag(want, "f16", S), S
        assert out.guards_intact()
    reps[3][lay.offset + 100] = float("nan")
    ctl = zs.device_ctl_new(1024.0, DEV)
    out = torch.empty(lay.count, dtype=torch.float16, device=DEV)
    zs.zero_reduce_shard_check_dev(out, reps, psi, n, rank, ctl)
    bias = zs.zero_bias_corrections(0.9, 0.999, 1, 4).to(DEV)
    zs.zero_scaler_update_dev(ctl, bias, 1)
    c = zs.device_ctl_read(ctl)
    assert c.found_inf == 1 and c.apply == 0 and c.scaler.loss_scale == 512.0
    log("reduce+check under device control: flags equal, the decision skips on the NaN")


def test_reduce_check_step_captured_in_a_graph():
    # a ZeRO-2 rank's whole device-resident step -- the reduce-scatter with the
    # check fused, the decision, the step -- captured once and replayed over new
    # replica gradients (one with a planted inf), each replay against the same
    # sequence run eagerly on a second copy of the state, bit for bit
    psi, n, rank = 400_003, 4, 1
    lay = zs.zero_shard_layout(psi, n, rank)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    bias = zs.zero_bias_corrections(0.9, 0.999, 1, 16).to(DEV)
    reps = make_replicas(psi, n, "f16", 61, std=1e-3 * 4096)
    master0 = torch.randn(lay.count, generator=torch.Generator().manual_seed(62)) * 0.02

    def state():
        return dict(master=master0.to(DEV), m=torch.zeros(lay.count, device=DEV),
                    v=torch.zeros(lay.count, device=DEV),
                    g=torch.empty(lay.count, dtype=torch.float16, device=DEV),
                    w=torch.zeros(lay.count, dtype=torch.float16, device=DEV),
                    ctl=zs.device_ctl_new(4096.0 * n, DEV))

    def enqueue(st):
        zs.zero_reduce_shard_check_dev(st["g"], reps, psi, n, rank, st["ctl"])
        zs.zero_scaler_update_dev(st["ctl"], bias, 1)
        zs.zero_adam_step_dev(st["w"], st["g"], st["master"], st["m"], st["v"], lay.count, 1, 0,
                              ctl=st["ctl"], **hp)

    E, G = state(), state()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        enqueue(G)
    torch.cuda.synchronize()
    fresh = make_replicas(psi, n, "f16", 63, std=1e-3 * 4096)
    for i in range(5):
        for k in range(n):
            reps[k].copy_(fresh[k])
            reps[k].mul_(1.0 + 0.125 * i)
        if i == 2:
            reps[0][lay.offset + 7] = float("inf")
        graph.replay()
        enqueue(E)
        torch.cuda.synchronize()
        for key in ("master", "m", "v", "g", "w"):
            a, b = E[key], G[key]
            iv = torch.int16 if a.dtype == torch.float16 else torch.int32
            assert torch.equal(a.view(iv), b.view(iv)), (i, key)
        ce, cg = zs.device_ctl_read(E["ctl"]), zs.device_ctl_read(G["ctl"])
        assert bytes(ce) == bytes(cg), i
        assert cg.found_inf == (1 if i == 2 else 0) and cg.apply == (0 if i == 2 else 1), i
    assert zs.device_ctl_read(G["ctl"]).scaler.step == 4
    del graph
    log("reduce+check -> decision -> step captured in a graph: every replay equals the eager run")
