"""GPU parity of the device-resident control path (check -> decision -> step
with S, t and the flag in device memory), against the host-driven oracle.

Ten steps of the ragged workload's schedule (inf/NaN on even steps) are
enqueued back to back without reading anything from the device, then the
arrays and the control block are compared with the oracle's sequence.
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
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)


def make_grads(count, steps, dtype, seed, bad_steps=(), std=1e-3):
    td = torch.float16 if dtype == "f16" else torch.bfloat16
    gs = []
    for t in range(1, steps + 1):
        g = synth.fill_normal_(torch.empty(count, dtype=td), std, seed + t)
        if t in bad_steps:
            synth.inject_nonfinite_(g, 3e-5, seed + 1000 + t)
        gs.append(g)
    return gs


def run_device(count, dtype, grads, S0, growth, phase=0, t_first=1, table_len=64, hp=HP):
    td = torch.float16 if dtype == "f16" else torch.bfloat16
    V = {k: GuardedView(count, td if k in ("g16", "w16") else torch.float32, phase, DEV)
         for k in ("g16", "w16", "master", "m", "v")}
    master0 = synth.fill_normal_(torch.empty(count), 0.02, 77)
    V["master"].view.copy_(master0.to(DEV))
    for k in ("m", "v", "w16"):
        V[k].view.zero_()
    ctl = zs.device_ctl_new(S0, DEV, growth_interval=growth)
    bias = zs.zero_bias_corrections(hp["beta1"], hp["beta2"], t_first, table_len).to(DEV)
    dgrads = [g.to(DEV) for g in grads]
    torch.cuda.synchronize()
    for g in dgrads:                 # no host read-back inside this loop
        V["g16"].view.copy_(g)
        zs.zero_overflow_check_dev(V["g16"].view, count, 1, 0, ctl)
        zs.zero_scaler_update_dev(ctl, bias, t_first)
        zs.zero_adam_step_dev(V["w16"].view, V["g16"].view, V["master"].view, V["m"].view,
                              V["v"].view, count, 1, 0, ctl=ctl, **hp)
    torch.cuda.synchronize()
    got = dict(master=f32(V["master"].view), m=f32(V["m"].view), v=f32(V["v"].view),
               w16=u16(V["w16"].view))
    assert all(gv.guards_intact() for gv in V.values())
    return got, zs.device_ctl_read(ctl), master0


def run_oracle(master0, grads, dtype, S0, growth, hp=HP):
    count = master0.numel()
    ref = dict(master=master0.numpy().copy(), m=np.zeros(count, np.float32),
               v=np.zeros(count, np.float32), w16=np.zeros(count, np.uint16))
    st = oracle.ScalerState(S0, growth_interval=growth)
    trace = []
    for g in grads:
        gh = u16(g)
        S = st.loss_scale
        flag, _ = oracle.overflow_check(gh, dtype, S)
        applied = oracle.policy(st, flag)
        if applied:
            oracle.adam_step(ref["w16"], gh, ref["master"], ref["m"], ref["v"], dtype,
                             step=st.step, loss_scale=S, **hp)
        trace.append((flag, applied, st.step, st.loss_scale))
    return ref, st, trace


@pytest.mark.parametrize("dtype,phase", [("f16", 0), ("f16", 3), ("bf16", 1)])
def test_device_schedule_matches_oracle(dtype, phase):
    count = 1_000_003
    grads = make_grads(count, 10, dtype, 500, bad_steps=(2, 4, 6, 8, 10))
    got, ctl, master0 = run_device(count, dtype, grads, 65536.0, 2000, phase=phase)
    ref, st, trace = run_oracle(master0, grads, dtype, 65536.0, 2000)
    log(f"oracle trace {trace}")
    assert [a for _, a, _, _ in trace] == [True, False] * 5
    assert (ctl.scaler.step, ctl.scaler.loss_scale, ctl.scaler.clean_steps) == \
        (st.step, st.loss_scale, st.clean_steps) == (5, 2048.0, 0)
    assert ctl.status == 0 and ctl.found_inf == 1 and ctl.apply == 0
    log("  device path", assert_close(got, ref, dtype, "device ctl"))


def test_device_growth_uses_scale_before_doubling():
    count = 300_001
    grads = make_grads(count, 6, "f16", 600, bad_steps=(3,))
    got, ctl, master0 = run_device(count, "f16", grads, 1024.0, 2)
    ref, st, trace = run_oracle(master0, grads, "f16", 1024.0, 2)
    log(f"oracle trace {trace}")
    assert (ctl.scaler.step, ctl.scaler.loss_scale) == (st.step, st.loss_scale)
    assert ctl.loss_scale_used == 2048.0   # the S in force for the last applied step
    assert_close(got, ref, "f16", "growth")


def test_device_step_outside_bias_table_is_skipped():
    count = 50_000
    grads = make_grads(count, 3, "f16", 700)
    # table covers t = 1 only: the second clean step falls outside it
    got, ctl, master0 = run_device(count, "f16", grads, 1.0, 2000, table_len=1)
    ref, st, _ = run_oracle(master0, grads[:1], "f16", 1.0, 2000)
    assert ctl.status == -4 and ctl.apply == 0 and ctl.scaler.step == 1
    assert_close(got, ref, "f16", "table range")


def test_device_nonpositive_scale_reads_as_overflow():
    count = 10_000
    g = make_grads(count, 1, "f16", 800)[0].to(DEV)
    for S in (0.0, -1.0, float("inf")):
        ctl = zs.device_ctl_new(S, DEV)
        zs.zero_overflow_check_dev(g, count, 1, 0, ctl)
        bias = zs.zero_bias_corrections(0.9, 0.999, 1, 4).to(DEV)
        zs.zero_scaler_update_dev(ctl, bias, 1)
        c = zs.device_ctl_read(ctl)
        assert c.found_inf == 1 and c.apply == 0 and c.status == -1 and c.scaler.step == 0


def test_decision_writes_the_reciprocals_the_step_multiplies_by():
    # after an applied decision the block holds S, bc1, bc2 and their FP64
    # reciprocals, each the correctly rounded 1/x (Python's float division is
    # IEEE round-to-nearest); S = 3 and 1000 take the reciprocal-product path
    count = 4096
    g = make_grads(count, 1, "f16", 900)[0].to(DEV)
    for S, b1, b2, t0 in ((65536.0, 0.9, 0.999, 1), (3.0, 0.9, 0.999, 1),
                          (1000.0, 0.95, 0.9999, 37), (2.0 ** -20, 0.5, 0.99, 5)):
        ctl = zs.device_ctl_new(S, DEV, step=t0 - 1)
        bias = zs.zero_bias_corrections(b1, b2, t0, 4).to(DEV)
        zs.zero_overflow_check_dev(g, count, 1, 0, ctl)
        zs.zero_scaler_update_dev(ctl, bias, t0)
        c = zs.device_ctl_read(ctl)
        host = zs.zero_bias_corrections(b1, b2, t0, 4).numpy()
        assert c.apply == 1 and c.status == 0 and c.scaler.step == t0
        assert (c.loss_scale_used, c.bc1, c.bc2) == (S, float(host[0]), float(host[4]))
        for got, x in ((c.rcp_loss_scale, S), (c.rcp_bc1, c.bc1), (c.rcp_bc2, c.bc2)):
            assert np.float64(got).view(np.uint64) == np.float64(1.0 / x).view(np.uint64), (S, x)
