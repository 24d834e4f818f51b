"""The device-controlled step captured once into a HIP graph and replayed.

With S, t and the skip flag in device memory, check -> decision -> step needs
no host read-back, so its launches (the step's as several consecutive launches
on a long shard) can be captured into one graph and replayed once per training
step.  Each replay is checked against the same
step run eagerly on a second copy of the state (bitwise: the same kernels on
the same inputs), with eager work and synchronisation between the replays,
and the final state against the oracle's host-driven sequence.
"""
import numpy as np
import pytest
import torch

import synth
import zero_sharded_mixed_shard_amd as zs
from gpu_util import GuardedView, assert_close, f32, log, u16
from test_gpu_c_device_ctl import HP, make_grads, run_oracle

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def state(count, dtype, phase, master0):
    td = torch.float16 if dtype == "f16" else torch.bfloat16
    V = {k: GuardedView(count, td if k in ("g16", "w16") else torch.float32, phase, DEV)
         for k in ("g16", "w16", "master", "m", "v")}
    V["master"].view.copy_(master0.to(DEV))
    for k in ("m", "v", "w16"):
        V[k].view.zero_()
    return V


def enqueue_step(V, count, ctl, bias, t_first):
    zs.zero_overflow_check_dev(V["g16"].view, count, 1, 0, ctl)
    zs.zero_scaler_update_dev(ctl, bias, t_first)
    zs.zero_adam_step_dev(V["w16"].view, V["g16"].view, V["master"].view, V["m"].view,
                          V["v"].view, count, 1, 0, ctl=ctl, **HP)


def host_state(V):
    return dict(master=f32(V["master"].view), m=f32(V["m"].view), v=f32(V["v"].view),
                w16=u16(V["w16"].view))


@pytest.mark.parametrize("dtype,phase,piece", [("f16", 0, 0), ("bf16", 3, 0), ("f16", 1, 7 * 2048)])
def test_graph_replays_match_eager_and_oracle(dtype, phase, piece):
    # piece: elements per step launch (0: the library's rule, one launch at this size;
    # 7 tiles: the step is captured as 70 consecutive launches, as long shards are)
    zs.zero_set_launch_piece(piece)
    try:
        graph_replays_case(dtype, phase)
    finally:
        torch.cuda.synchronize()
        zs.zero_set_launch_piece(0)


def graph_replays_case(dtype, phase):
    count, steps, S0 = 1_000_003, 8, 65536.0
    grads = make_grads(count, steps, dtype, 900, bad_steps=(3, 6))
    dgrads = [g.to(DEV) for g in grads]
    master0 = synth.fill_normal_(torch.empty(count), 0.02, 91)
    bias = zs.zero_bias_corrections(HP["beta1"], HP["beta2"], 1, 64).to(DEV)

    E = state(count, dtype, phase, master0)        # eager copy
    G = state(count, dtype, phase, master0)        # graph copy
    ctl_e = zs.device_ctl_new(S0, DEV)
    ctl_g = zs.device_ctl_new(S0, DEV)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        enqueue_step(G, count, ctl_g, bias, 1)
    torch.cuda.synchronize()
    # capturing runs nothing: the graph's state is still the initial one
    assert zs.device_ctl_read(ctl_g).scaler.step == 0
    assert np.array_equal(f32(G["master"].view), master0.numpy())

    for t, g in enumerate(dgrads, start=1):
        G["g16"].view.copy_(g)
        graph.replay()
        E["g16"].view.copy_(g)
        enqueue_step(E, count, ctl_e, bias, 1)
        torch.cuda.synchronize()
        he, hg = host_state(E), host_state(G)
        for k in he:
            assert np.array_equal(he[k].view(np.uint8), hg[k].view(np.uint8)), (dtype, t, k)
        assert bytes(zs.device_ctl_read(ctl_e)) == bytes(zs.device_ctl_read(ctl_g)), (dtype, t)

    ref, st, trace = run_oracle(master0, grads, dtype, S0, 2000)
    assert [a for _, a, _, _ in trace] == [True, True, False, True, True, False, True, True]
    c = zs.device_ctl_read(ctl_g)
    assert (c.scaler.step, c.scaler.loss_scale) == (st.step, st.loss_scale) == (6, 16384.0)
    log(f"  graph x{steps} {dtype}", assert_close(host_state(G), ref, dtype, "graph replay"))
    assert all(v.guards_intact() for v in G.values())
    del graph


def test_graph_captures_the_allocation_free_check():
    # the allocation-free check (flag and sum of squares, its partial sums in the
    # library's fixed array) captured once and replayed over new gradients, with an
    # eager call of another size between replays rewriting the shared array: every
    # replay equals the workspace form on the same gradients, bit for bit
    count, S = 1_000_003, 3.0
    g = GuardedView(count, torch.float16, 1, DEV)
    other = torch.empty(70_001, dtype=torch.bfloat16, device=DEV).fill_(0.5)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    ssq = torch.zeros(1, device=DEV)
    oflag = torch.zeros(1, dtype=torch.int32, device=DEV)
    ossq = torch.zeros(1, device=DEV)
    wflag = torch.zeros(1, dtype=torch.int32, device=DEV)
    wssq = torch.zeros(1, device=DEV)
    parts = torch.empty(zs.SUMSQ_PARTIALS, dtype=torch.float64, device=DEV)
    g.view.copy_(synth.fill_normal_(torch.empty(count, dtype=torch.float16), 1e-2, 95).to(DEV))
    zs.zero_overflow_check_noalloc(g.view, count, 1, 0, S, flag, ssq)   # before capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        zs.zero_overflow_check_noalloc(g.view, count, 1, 0, S, flag, ssq)
    torch.cuda.synchronize()
    for i in range(5):
        grads = synth.fill_normal_(torch.empty(count, dtype=torch.float16), 1e-2, 96 + i)
        if i == 3:
            grads[count // 2] = float("inf")
        g.view.copy_(grads.to(DEV))
        graph.replay()
        zs.zero_overflow_check_noalloc(other, other.numel(), 1, 0, 1.0, oflag, ossq)
        torch.cuda.synchronize()
        got = (int(flag.item()), int(ssq.view(torch.int32).item()))
        zs.zero_overflow_check(g.view, count, 1, 0, S, wflag, wssq, parts)
        torch.cuda.synchronize()
        want = (int(wflag.item()), int(wssq.view(torch.int32).item()))
        assert got == want, (i, got, want)
        assert got[0] == (1 if i == 3 else 0)
        assert float(ossq.item()) == 0.25 * other.numel() and int(oflag.item()) == 0
    assert g.guards_intact()
    del graph
