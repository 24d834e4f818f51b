"""Sharded checkpoint resume on the GPU: 3 steps on 8 device shards, each rank
saves its slice, the run resumes on 5 shards (resharded read) with the saved
step counter and loss scale, 2 more steps, and the result equals the oracle's
uninterrupted 5 steps on the unsharded buffer bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import synth
import zero_sharded_mixed_shard_amd as zs
from gpu_util import assert_close, f32, log, u16

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def test_resume_on_five_ranks_from_eight(tmp_path):
    psi, S = 2_000_003, 1024.0
    grads = [synth.fill_normal_(torch.empty(psi, dtype=torch.bfloat16), 1e-3 * S, 7000 + t)
             for t in range(5)]
    master0 = synth.fill_normal_(torch.empty(psi), 0.02, 7100)
    ref = [np.zeros(psi, np.uint16), master0.numpy().copy(), np.zeros(psi, np.float32),
           np.zeros(psi, np.float32)]
    for t in range(1, 6):
        oracle.adam_step(ref[0], u16(grads[t - 1]), ref[1], ref[2], ref[3], "bf16", step=t,
                         loss_scale=S, **HP)

    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    paths = []
    for k in range(8):
        lay = zs.zero_shard_layout(psi, 8, k)
        sl = slice(lay.offset, lay.offset + lay.count)
        w = torch.zeros(lay.count, dtype=torch.bfloat16, device=DEV)
        mast = master0[sl].to(DEV)
        m = torch.zeros(lay.count, device=DEV)
        v = torch.zeros(lay.count, device=DEV)
        sc = zs.Scaler(S)
        for t in range(1, 4):
            g = grads[t - 1][sl].to(DEV)
            zs.zero_overflow_check(g, psi, 8, k, sc.loss_scale, flag)
            S_used = sc.loss_scale
            assert zs.zero_scaler_update(sc, int(flag.item()))
            zs.zero_adam_step(w, g, mast, m, v, psi, 8, k, step=sc.step, loss_scale=S_used, **HP)
        p = str(tmp_path / f"rank{k}.zshard")
        zs.zero_ckpt_write(p, psi, 8, k, torch.bfloat16, sc, u16(w), f32(mast), f32(m), f32(v))
        zs.zero_ckpt_verify(p)
        paths.append(p)
    log("saved 8 shards")

    got = {key: [] for key in ("w16", "master", "m", "v")}
    for r in range(5):
        info = zs.zero_ckpt_read_info(paths[0])
        sc = zs.Scaler(info.scaler.loss_scale, info.scaler.growth_interval, info.scaler.step)
        sc.clean_steps = info.scaler.clean_steps
        assert sc.step == 3
        lay = zs.zero_shard_layout(psi, 5, r)
        sl = slice(lay.offset, lay.offset + lay.count)
        hw, hm, hmm, hv = zs.zero_ckpt_read_resharded(paths, psi, 5, r)
        w = torch.from_numpy(hw.view(np.int16).copy()).view(torch.bfloat16).to(DEV)
        mast, m, v = (torch.from_numpy(a).to(DEV) for a in (hm, hmm, hv))
        for t in range(4, 6):
            g = grads[t - 1][sl].to(DEV)
            zs.zero_overflow_check(g, psi, 5, r, sc.loss_scale, flag)
            S_used = sc.loss_scale
            assert zs.zero_scaler_update(sc, int(flag.item()))
            assert sc.step == t
            zs.zero_adam_step(w, g, mast, m, v, psi, 5, r, step=sc.step, loss_scale=S_used, **HP)
        torch.cuda.synchronize()
        got["w16"].append(u16(w))
        got["master"].append(f32(mast))
        got["m"].append(f32(m))
        got["v"].append(f32(v))
    got = {k: np.concatenate(v) for k, v in got.items()}
    log("  resumed 8 -> 5", assert_close(got, dict(w16=ref[0], master=ref[1], m=ref[2], v=ref[3]),
                                        "bf16", "resume"))
