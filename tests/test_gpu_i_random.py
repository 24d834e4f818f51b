"""Seeded random parity sweep: check -> decision -> step against the oracle.

Each case draws a shard size (1 to ~300k elements, biased toward tile and
line boundaries), view phases (all equal, or mixed: the element-wise kernel),
a 16-bit format, hyperparameters (including beta = 0, eps = 0, wd = 0 and
negative lr), a loss scale (powers of two and not), a gradient spread from
deep in the FP16 subnormal range to values that overflow after unscaling,
and sometimes planted inf/NaN.  The flag, the skip-or-apply decision and
the state after up to three steps must meet the parity bar.
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


def test_random_sweep_matches_oracle():
    rng = np.random.default_rng(20261202)
    stats = {"cases": 0, "skipped_steps": 0, "applied_steps": 0, "mixed_phase": 0}
    for case in range(N_CASES):
        count, phases, dtype, hp, S, std, inject, steps = draw_case(rng)
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
        assert_close(got, ref, dtype, f"case {case}: count={count} phases={phases} {dtype} "
                                      f"hp={hp} S={S} std={std:.3g}")
        assert all(x.guards_intact() for x in V.values()), case
        stats["cases"] += 1
        stats["mixed_phase"] += len(set(phases.values())) > 1
    log(f"random sweep: {stats}")
    assert stats["skipped_steps"] > 0 and stats["applied_steps"] > 0 and stats["mixed_phase"] > 0
