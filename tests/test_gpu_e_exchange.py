"""GPU parity of the one-GPU exchange stand-ins against the oracle.

* zero_reduce_shard: every rank's chunk of the FP32 sum of n replicas, for
  each input/output format, n from 1 to 64, ragged sizes and misaligned views;
* zero_gather_shards: every element lands at its flat index, the padded tail
  and guards stay untouched;
* reduce-scatter then all-gather equals the all-reduce (the oracle's
  element-wise sum of the full replicas);
* a whole data-parallel step on one GPU: the n replicas' gradients are
  reduce-scattered, each rank checks (separately, or fused into the
  reduce-scatter) and steps its shard, the 16-bit shards are all-gathered,
  and the result equals the unsharded update of the summed gradients, bit
  for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import zero_sharded_mixed_shard_amd as zs
from gpu_util import GuardedView, SENT16, assert_close, f32, log, u16

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TD = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def host(t: torch.Tensor) -> np.ndarray:
    return f32(t) if t.dtype == torch.float32 else u16(t)


def make_replicas(psi, n, fmt, seed, phase=0, std=1e-2):
    """n device replicas of psi elements; the returned tensors are views at `phase`."""
    reps = []
    for k in range(n):
        x = synth.fill_normal_(torch.empty(psi, dtype=TD[fmt]), std, seed + k)
        buf = torch.empty(psi + 8, dtype=TD[fmt], device=DEV)
        view = buf[phase:phase + psi]
        view.copy_(x.to(DEV))
        reps.append(view)
    return reps


@pytest.mark.parametrize("in_fmt,out_fmt", [("f16", "f32"), ("f16", "f16"), ("bf16", "bf16"),
                                            ("f32", "f32"), ("bf16", "f32"), ("f32", "f16")])
def test_reduce_shard_matches_oracle(in_fmt, out_fmt):
    for psi, n in ((1, 1), (10, 8), (1000, 8), (100_003, 8), (65_537, 3), (4096 * 64 + 5, 64)):
        for phase in (0, 1):
            reps = make_replicas(psi, n, in_fmt, 17 * psi + n, phase)
            hreps = [host(r) for r in reps]
            for rank in sorted({0, n // 2, n - 1}):
                lay = zs.zero_shard_layout(psi, n, rank)
                out = GuardedView(lay.count, TD[out_fmt], (rank + phase) % 4, DEV)
                zs.zero_reduce_shard(out.view, reps, psi, n, rank)
                ref = oracle.reduce_shard(hreps, in_fmt, out_fmt, psi, n, rank)
                got = host(out.view)
                assert np.array_equal(got.view(np.uint8), ref.view(np.uint8)), \
                    (in_fmt, out_fmt, psi, n, rank, phase)
                assert out.guards_intact()
    log(f"reduce {in_fmt}->{out_fmt}: bitwise")


@pytest.mark.parametrize("fmt", ["f16", "f32"])
def test_gather_and_identity_with_all_reduce(fmt):
    for psi, n in ((10, 8), (1003, 8), (1_000_003, 8), (777, 64), (5, 1)):
        reps = make_replicas(psi, n, fmt, 31 * psi + n)
        hreps = [host(r) for r in reps]
        shards = []
        for k in range(n):
            lay = zs.zero_shard_layout(psi, n, k)
            if lay.count == 0:
                shards.append(None)
                continue
            s = torch.empty(lay.count + 3, dtype=TD[fmt], device=DEV)[k % 3:k % 3 + lay.count]
            zs.zero_reduce_shard(s, reps, psi, n, k)
            shards.append(s)
        padded = zs.zero_shard_layout(psi, n, 0).padded_total
        full = GuardedView(padded, TD[fmt], 0, DEV)
        zs.zero_gather_shards(full.view, shards, psi, n)
        got = host(full.view)
        allreduce = np.zeros(psi, np.float32)
        for h in hreps:
            allreduce = allreduce + (h if fmt == "f32" else oracle.decode16(h, fmt))
        want = allreduce if fmt == "f32" else oracle.encode16(allreduce, fmt)
        assert np.array_equal(got[:psi].view(np.uint8), want.view(np.uint8)), (psi, n)
        # the padding of the flat buffer and the guards are not written
        tail = got[psi:]
        if fmt == "f32":
            assert np.all(tail.view(np.uint32) == 0x7FC0DEAD)
        else:
            assert np.all(tail == SENT16)
        assert full.guards_intact()
        # the oracle's all-gather of the host shards agrees
        hshards = [np.zeros(0, got.dtype) if s is None else host(s) for s in shards]
        ref_full = np.zeros(psi, got.dtype)
        oracle.gather_shards(hshards, psi, n, ref_full)
        assert np.array_equal(ref_full.view(np.uint8), got[:psi].view(np.uint8))
    log(f"gather {fmt}: bitwise; RS + AG == AR")


@pytest.mark.parametrize("fused", [False, True])
def test_data_parallel_step_on_one_gpu(fused):
    # ZeRO-2 step with n = 8 simulated ranks on one GPU: 16-bit gradients of
    # 8 replicas -> reduce-scatter (FP16 out, the sum carries 8x the loss
    # scale) -> per-rank check + step on its shard -> all-gather of the 16-bit
    # weights.  Equals the unsharded step on the all-reduced gradients.  fused:
    # the check rides on the reduce-scatter (zero_reduce_shard_check).
    psi, n = 1_000_003, 8
    S = 1024.0 * n        # loss scale times n: the reduce leaves the SUM (R-11)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    master0 = synth.fill_normal_(torch.empty(psi), 0.02, 4242)
    shards = []
    for k in range(n):
        lay = zs.zero_shard_layout(psi, n, k)
        sl = slice(lay.offset, lay.offset + lay.count)
        shards.append(dict(master=master0[sl].clone().to(DEV),
                           m=torch.zeros(lay.count, device=DEV),
                           v=torch.zeros(lay.count, device=DEV),
                           g=torch.empty(lay.count, dtype=torch.float16, device=DEV),
                           w=torch.zeros(lay.count, dtype=torch.float16, device=DEV)))
    full_w = torch.zeros(psi, dtype=torch.float16, device=DEV)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    ref = dict(master=master0.numpy().copy(), m=np.zeros(psi, np.float32),
               v=np.zeros(psi, np.float32), w16=np.zeros(psi, np.uint16))
    for t in (1, 2, 3):
        reps = make_replicas(psi, n, "f16", 5000 + 10 * t, std=1e-3 * 1024)
        for k in range(n):
            sh = shards[k]
            if fused:
                zs.zero_reduce_shard_check(sh["g"], reps, psi, n, k, S, flag)
            else:
                zs.zero_reduce_shard(sh["g"], reps, psi, n, k)
                zs.zero_overflow_check(sh["g"], psi, n, k, S, flag)
            zs.zero_adam_step(sh["w"], sh["g"], sh["master"], sh["m"], sh["v"], psi, n, k,
                              step=t, loss_scale=S, found_inf=flag, **hp)
        zs.zero_gather_shards(full_w, [sh["w"] for sh in shards], psi, n)
        # oracle: all-reduce (sum of replicas, FP32, rank order, rounded to FP16), then step
        hreps = [u16(r) for r in reps]
        g_sum = oracle.encode16(sum_f32([oracle.decode16(h, "f16") for h in hreps]), "f16")
        assert oracle.overflow_check(g_sum, "f16", S)[0] == 0
        oracle.adam_step(ref["w16"], g_sum, ref["master"], ref["m"], ref["v"], "f16", step=t,
                         loss_scale=S, **hp)
    torch.cuda.synchronize()
    got = dict(master=np.concatenate([f32(sh["master"]) for sh in shards]),
               m=np.concatenate([f32(sh["m"]) for sh in shards]),
               v=np.concatenate([f32(sh["v"]) for sh in shards]), w16=u16(full_w))
    log(f"  RS -> step -> AG (check fused: {fused})", assert_close(got, ref, "f16", "dp step"))


def sum_f32(arrays):
    acc = np.zeros(arrays[0].size, np.float32)
    for a in arrays:
        acc = acc + a
    return acc


@pytest.mark.parametrize("fmt", ["f16", "f32"])
def test_in_place_reduce_scatter_and_all_gather(fmt):
    # In place, as collective libraries allow it: rank k's reduce-scatter result
    # overwrites its own chunk of replica k, and the all-gather reads shards that
    # already sit at their places in the full buffer (here: even ranks) beside
    # shards held elsewhere (odd ranks).  Partial overlaps are rejected.
    psi, n = 100_003, 4
    reps = make_replicas(psi, n, fmt, 4100 + len(fmt))
    hreps = [host(r) for r in reps]
    want = [oracle.reduce_shard(hreps, fmt, fmt, psi, n, k) for k in range(n)]
    lays = [zs.zero_shard_layout(psi, n, k) for k in range(n)]
    for k, lay in enumerate(lays):
        zs.zero_reduce_shard(reps[k][lay.offset:lay.offset + lay.count], reps, psi, n, k)
    for k, lay in enumerate(lays):
        got = host(reps[k][lay.offset:lay.offset + lay.count])
        assert np.array_equal(got.view(np.uint8), want[k].view(np.uint8)), (fmt, k)
    full = GuardedView(lays[0].padded_total, TD[fmt], 0, DEV)
    shards = []
    for k, lay in enumerate(lays):
        if k % 2 == 0:
            s = full.view[lay.offset:lay.offset + lay.count]
        else:
            s = torch.empty(lay.count, dtype=TD[fmt], device=DEV)
        s.copy_(reps[k][lay.offset:lay.offset + lay.count])
        shards.append(s)
    zs.zero_gather_shards(full.view, shards, psi, n)
    got = host(full.view)[:psi]
    assert np.array_equal(got.view(np.uint8), np.concatenate(want).view(np.uint8))
    assert full.guards_intact()
    # a shard overlapping the full buffer anywhere but at its place
    bad = list(shards)
    bad[1] = full.view[7:7 + lays[1].count]
    with pytest.raises(zs.ZeroError):
        zs.zero_gather_shards(full.view, bad, psi, n)
    lay0 = lays[0]
    with pytest.raises(zs.ZeroError):      # the output straddling replica 1's chunk
        zs.zero_reduce_shard(reps[1][lay0.offset + 3:lay0.offset + 3 + lay0.count], reps, psi, n, 0)
    log(f"in-place reduce-scatter / all-gather {fmt}: bitwise")
