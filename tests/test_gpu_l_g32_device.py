"""The device-resident control path over FP32 gradients: micro-batches
accumulated in FP32, then check -> decision -> step with S, t and the flag in
device memory, against the oracle's host-driven sequence.

An overflow is planted in one micro-batch of some steps; nothing is read back
inside the loop.  The same training step -- k accumulations, the check, the
decision and the step -- is then captured once into a HIP graph and replayed
per step, each replay checked bit for bit against the same step run eagerly on
a second copy of the state (with eager work and synchronisation between
replays), and the final state against the oracle.  Both run with the check as
its own pass and fused into the last micro-batch's accumulate.
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
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def micro_batches(count, steps, k, dtype, seed, bad_steps):
    out = []
    for t in range(1, steps + 1):
        mbs = []
        for j in range(k):
            g = synth.fill_normal_(torch.empty(count, dtype=TD[dtype]), 1e-3, seed + 10 * t + j)
            if t in bad_steps and j == k - 1:
                synth.inject_nonfinite_(g, 3e-5, seed + 5000 + t)
            mbs.append(g)
        out.append(mbs)
    return out


class State:
    def __init__(self, count, dtype, phase, master0):
        self.V = {k: GuardedView(count, TD[dtype] if k == "w16" else torch.float32, phase, DEV)
                  for k in ("acc", "w16", "master", "m", "v")}
        self.V["master"].view.copy_(master0.to(DEV))
        for k in ("m", "v", "w16"):
            self.V[k].view.zero_()

    def host(self):
        return {k: (u16 if k == "w16" else f32)(self.V[k].view) for k in ("master", "m", "v", "w16")}

    def intact(self):
        return all(v.guards_intact() for v in self.V.values())


def enqueue_training_step(st, mb_views, count, ctl, bias, fused=False):
    # fused: the last micro-batch's accumulate carries the check of the result
    V = st.V
    for j, g in enumerate(mb_views):
        if fused and j == len(mb_views) - 1:
            zs.zero_grad_accumulate_check_dev(V["acc"].view, g, count, 1, 0, first=(j == 0),
                                              ctl=ctl)
        else:
            zs.zero_grad_accumulate(V["acc"].view, g, count, 1, 0, first=(j == 0))
    if not fused:
        zs.zero_overflow_check_g32_dev(V["acc"].view, count, 1, 0, ctl)
    zs.zero_scaler_update_dev(ctl, bias, 1)
    zs.zero_adam_step_g32_dev(V["w16"].view, V["acc"].view, V["master"].view, V["m"].view,
                              V["v"].view, count, 1, 0, ctl=ctl, **HP)


def run_oracle(master0, batches, dtype, S0, growth):
    count = master0.numel()
    ref = dict(master=master0.numpy().copy(), m=np.zeros(count, np.float32),
               v=np.zeros(count, np.float32), w16=np.zeros(count, np.uint16))
    sc = oracle.ScalerState(S0, growth_interval=growth)
    racc = np.zeros(count, np.float32)
    trace = []
    for mbs in batches:
        for j, g in enumerate(mbs):
            oracle.grad_accumulate(racc, u16(g), dtype, first=(j == 0))
        S = sc.loss_scale
        flag, _ = oracle.overflow_check_g32(racc, S)
        applied = oracle.policy(sc, flag)
        if applied:
            oracle.adam_step_g32(ref["w16"], racc, ref["master"], ref["m"], ref["v"], dtype,
                                 step=sc.step, loss_scale=S, **HP)
        trace.append((flag, applied))
    return ref, sc, trace


@pytest.mark.parametrize("dtype,phase,fused", [("f16", 0, False), ("bf16", 3, False),
                                               ("f16", 1, True), ("bf16", 0, True)])
def test_device_controlled_fp32_gradient_schedule(dtype, phase, fused):
    count, steps, k, S0, growth = 300_007, 8, 3, 1024.0, 2
    batches = micro_batches(count, steps, k, dtype, 61_000, bad_steps=(3, 6))
    master0 = synth.fill_normal_(torch.empty(count), 0.02, 61_900)
    st = State(count, dtype, phase, master0)
    mb = [GuardedView(count, TD[dtype], phase, DEV) for _ in range(k)]
    ctl = zs.device_ctl_new(S0, DEV, growth_interval=growth)
    bias = zs.zero_bias_corrections(HP["beta1"], HP["beta2"], 1, 32).to(DEV)
    dev_batches = [[g.to(DEV) for g in mbs] for mbs in batches]
    torch.cuda.synchronize()
    for mbs in dev_batches:            # no host read-back inside this loop
        for view, g in zip(mb, mbs):
            view.view.copy_(g)
        enqueue_training_step(st, [m.view for m in mb], count, ctl, bias, fused=fused)
    torch.cuda.synchronize()
    ref, sc, trace = run_oracle(master0, batches, dtype, S0, growth)
    assert [a for _, a in trace] == [True, True, False, True, True, False, True, True]
    c = zs.device_ctl_read(ctl)
    assert (c.scaler.step, c.scaler.loss_scale, c.scaler.clean_steps) == \
        (sc.step, sc.loss_scale, sc.clean_steps)
    assert c.status == 0 and c.apply == 1
    log(f"  FP32-gradient device schedule {dtype} fused={fused}: t {c.scaler.step}, "
        f"S {c.scaler.loss_scale}",
        assert_close(st.host(), ref, dtype, "g32 device schedule"))
    assert st.intact() and all(m.guards_intact() for m in mb)


@pytest.mark.parametrize("fused", [False, True])
def test_fp32_gradient_training_step_graph_replays(fused):
    dtype, count, steps, k, S0, growth = "f16", 1_000_003, 6, 2, 65536.0, 2
    batches = micro_batches(count, steps, k, dtype, 62_000, bad_steps=(4,))
    master0 = synth.fill_normal_(torch.empty(count), 0.02, 62_900)
    bias = zs.zero_bias_corrections(HP["beta1"], HP["beta2"], 1, 32).to(DEV)
    E, G = State(count, dtype, 0, master0), State(count, dtype, 0, master0)
    ctl_e = zs.device_ctl_new(S0, DEV, growth_interval=growth)
    ctl_g = zs.device_ctl_new(S0, DEV, growth_interval=growth)
    mb = [torch.empty(count, dtype=TD[dtype], device=DEV) for _ in range(k)]
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        enqueue_training_step(G, mb, count, ctl_g, bias, fused=fused)
    torch.cuda.synchronize()
    assert zs.device_ctl_read(ctl_g).scaler.step == 0          # capture ran nothing

    for t, mbs in enumerate(batches, start=1):
        for view, g in zip(mb, mbs):
            view.copy_(g.to(DEV))
        graph.replay()
        torch.cuda.synchronize()
        enqueue_training_step(E, mb, count, ctl_e, bias, fused=fused)
        torch.cuda.synchronize()
        he, hg = E.host(), G.host()
        for key in he:
            assert np.array_equal(he[key].view(np.uint8), hg[key].view(np.uint8)), (t, key)
        assert np.array_equal(f32(E.V["acc"].view).view(np.uint32),
                              f32(G.V["acc"].view).view(np.uint32)), t
        assert bytes(zs.device_ctl_read(ctl_e)) == bytes(zs.device_ctl_read(ctl_g)), t

    ref, sc, trace = run_oracle(master0, batches, dtype, S0, growth)
    assert [a for _, a in trace] == [True, True, True, False, True, True]
    c = zs.device_ctl_read(ctl_g)
    assert (c.scaler.step, c.scaler.loss_scale) == (sc.step, sc.loss_scale)
    log(f"  FP32-gradient training step, graph x{steps}, fused={fused}",
        assert_close(G.host(), ref, dtype, "g32 graph"))
    assert G.intact()
    del graph
