"""GPU parity on the six workloads at their real sizes.

C1 (1M params, rank 3 of 8)    three ZeRO layouts, every element, all agree bitwise
C2 (GPT-2-small shapes, N=8)  every element of all 8 ranks for 10 steps, and the
                              concatenated shards equal the unsharded (N=1) update
C3 (7.5e9, N=8, BF16)         rank 1's 937.5M-element shard, 20 warm steps: the first step
                              against the oracle at every element, all 20 on sampled windows,
                              and invariants at every element
C4 (1e10, N=1, 160 GB)        the whole buffer, 5 steps: the first step against the oracle at
                              every element (indices past 2^32 included), all 5 on windows up
                              to the last element, invariants at every element, flag
                              property at a far position
C5 (8,810,000,003, N=64)      rank 63's ragged shard (61 padding elements, start = 5 mod 8),
                              10 steps with inf/NaN injection on even steps: every flag,
                              every element, S halving and t bit-exact against the oracle
C6 (1.5e9, N=1, BF16, 24 GB)  the whole buffer, 10 steps: the last step against the oracle at
                              every element, all 10 on sampled windows, and invariants at
                              every element
(invariants: w16 = RNE16(master) bitwise, v >= 0, master, m and v finite)

Inputs come from `synth` (seeded); expected values only from `oracle`.
"""
import gc

import time

import numpy as np
import pytest
import torch

import oracle
import synth
import zero_sharded_mixed_shard_amd as zs
from gpu_util import GuardedView, SENT16, assert_close, f32, hp_of, log, u16

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def flag_buf():
    return torch.zeros(1, dtype=torch.int32, device=DEV)


def host_state(master, m, v, w16):
    return dict(master=master, m=m, v=v, w16=w16)


# ---------------------------------------------------------------------------
# C1: three layouts of rank 3's shard
# ---------------------------------------------------------------------------

def test_c1_three_zero_layouts():
    w = synth.WORKLOADS[1]
    psi, n, r = w.psi, w.n, 3
    lay = zs.zero_shard_layout(psi, n, r)
    cnt, off = lay.count, lay.offset
    hp = hp_of(w)
    master0 = synth.fill_normal_(torch.empty(cnt), w.master_std, synth.seed_of(1, 2))
    grads = [synth.fill_normal_(torch.empty(psi, dtype=torch.float16), w.grad_std,
                                synth.seed_of(1, 1, t)) for t in range(1, w.steps + 1)]

    def fresh_local():
        return (master0.to(DEV), torch.zeros(cnt, device=DEV), torch.zeros(cnt, device=DEV))

    results = {}
    for name in ("zero1", "zero2", "zero3"):
        log(f"C1 layout {name}")
        master, m, v = fresh_local()
        full_w = GuardedView(psi, torch.float16, 0, DEV)   # replicated working weights
        full_g = GuardedView(psi, torch.float16, 0, DEV)   # replicated gradients (ZeRO-1)
        if name == "zero3":
            w16 = torch.zeros(cnt, dtype=torch.float16, device=DEV)
        else:
            w16 = full_w.view[off:off + cnt]
        flag = flag_buf()
        for t in range(1, w.steps + 1):
            if name == "zero1":
                full_g.view.copy_(grads[t - 1].to(DEV))
                g16 = full_g.view[off:off + cnt]
            else:
                g16 = grads[t - 1][off:off + cnt].to(DEV)
            zs.zero_overflow_check(g16, psi, n, r, w.loss_scale, flag)
            assert flag.item() == 0
            zs.zero_adam_step(w16, g16, master, m, v, psi, n, r, step=t,
                              loss_scale=w.loss_scale, found_inf=flag, **hp)
        torch.cuda.synchronize()
        results[name] = dict(master=f32(master), m=f32(m), v=f32(v), w16=u16(w16))
        if name != "zero3":
            # the rest of the replicated buffer is never written
            outside = np.concatenate([u16(full_w.view[:off]), u16(full_w.view[off + cnt:])])
            assert np.all(outside == SENT16)
            assert full_w.guards_intact()
        if name == "zero1":
            assert np.array_equal(u16(full_g.view), synth.to_numpy_u16(grads[-1]))

    ref = host_state(master0.numpy().copy(), np.zeros(cnt, np.float32),
                     np.zeros(cnt, np.float32), np.zeros(cnt, np.uint16))
    for t in range(1, w.steps + 1):
        g = synth.to_numpy_u16(grads[t - 1][off:off + cnt])
        assert oracle.overflow_check(g, "f16", w.loss_scale)[0] == 0
        oracle.adam_step(ref["w16"], g, ref["master"], ref["m"], ref["v"], "f16", step=t,
                         loss_scale=w.loss_scale, **hp)
    for name, got in results.items():
        log(f"  {name}", assert_close(got, ref, "f16", name))
    for k in ("master", "m", "v", "w16"):
        assert np.array_equal(results["zero1"][k], results["zero2"][k])
        assert np.array_equal(results["zero1"][k], results["zero3"][k])


# ---------------------------------------------------------------------------
# C2: GPT-2-small-shaped flat buffer, all 8 ranks, ZeRO-2 layout
# ---------------------------------------------------------------------------

def test_c2_gpt2_shapes_all_ranks_and_unsharded_equivalence():
    w = synth.WORKLOADS[2]
    shapes = synth.gpt2_small_shapes()
    sizes = [int(np.prod(s)) for _, s in shapes]
    assert len(shapes) == 148 and sum(sizes) == w.psi == 124_439_808
    psi, n, hp, S = w.psi, w.n, hp_of(w), w.loss_scale
    lays = [zs.zero_shard_layout(psi, n, r) for r in range(n)]
    assert all(l.pad == 0 for l in lays)           # 8 divides psi: no padding
    # tensors that straddle a shard boundary: the flat kernel ignores them
    bounds = np.cumsum([0] + sizes)
    straddle = [shapes[i][0] for i in range(148)
                if bounds[i] // lays[0].shard != (bounds[i + 1] - 1) // lays[0].shard]
    log(f"C2 shard {lays[0].shard}; tensors across shard boundaries: {straddle}")

    master_full = synth.fill_normal_(torch.empty(psi, device=DEV), w.master_std,
                                     synth.seed_of(2, 2))
    w16_full = torch.zeros(psi, dtype=torch.float16, device=DEV)   # replicated (ZeRO-2)
    shards = []
    for l in lays:
        sl = slice(l.offset, l.offset + l.count)
        shards.append(dict(master=master_full[sl].clone(),
                           m=torch.zeros(l.count, device=DEV), v=torch.zeros(l.count, device=DEV),
                           g16=torch.empty(l.count, dtype=torch.float16, device=DEV)))
    one = dict(master=master_full.clone(), m=torch.zeros(psi, device=DEV),
               v=torch.zeros(psi, device=DEV), w16=torch.zeros(psi, dtype=torch.float16,
                                                              device=DEV))
    ref = host_state(f32(master_full), np.zeros(psi, np.float32), np.zeros(psi, np.float32),
                     np.zeros(psi, np.uint16))
    del master_full
    flag = flag_buf()
    g_full = torch.empty(psi, dtype=torch.float16, device=DEV)
    for t in range(1, w.steps + 1):
        synth.fill_normal_(g_full, w.grad_std, synth.seed_of(2, 1, t))
        for r, l in enumerate(lays):
            sh = shards[r]
            sh["g16"].copy_(g_full[l.offset:l.offset + l.count])
            zs.zero_overflow_check(sh["g16"], psi, n, r, S, flag)
            zs.zero_adam_step(w16_full[l.offset:l.offset + l.count], sh["g16"], sh["master"],
                              sh["m"], sh["v"], psi, n, r, step=t, loss_scale=S,
                              found_inf=flag, **hp)
        zs.zero_adam_step(one["w16"], g_full, one["master"], one["m"], one["v"], psi, 1, 0,
                          step=t, loss_scale=S, **hp)
        g_host = u16(g_full)
        assert oracle.overflow_flag_mt(g_host, "f16", S) == 0
        assert flag.item() == 0
        oracle.adam_step_mt(ref["w16"], g_host, ref["master"], ref["m"], ref["v"], "f16",
                            step=t, loss_scale=S, **hp)
        log(f"  step {t} done")
    torch.cuda.synchronize()
    got = dict(master=np.concatenate([f32(s["master"]) for s in shards]),
               m=np.concatenate([f32(s["m"]) for s in shards]),
               v=np.concatenate([f32(s["v"]) for s in shards]), w16=u16(w16_full))
    log("  vs oracle", assert_close(got, ref, "f16", "C2"))
    unsharded = dict(master=f32(one["master"]), m=f32(one["m"]), v=f32(one["v"]),
                     w16=u16(one["w16"]))
    for k in got:
        assert np.array_equal(got[k].view(np.uint8), unsharded[k].view(np.uint8)), k


# ---------------------------------------------------------------------------
# windows: full-size shards checked on sampled ranges the oracle can follow
# ---------------------------------------------------------------------------

def windows_of(count, rng, n_random=24, width=8192, edge=4096):
    w = [(0, min(edge, count)), (max(0, count - edge), count)]
    for s in rng.integers(0, max(1, count - width), n_random):
        w.append((int(s), int(min(count, s + width))))
    if count > 2 ** 32 + width:
        w.append((2 ** 32 - width // 2, 2 ** 32 + width // 2))
        w.append((2 ** 33 - 3, 2 ** 33 + width))
    return sorted(w)


def full_buffer_invariants(master, m, v, w16, what, chunk=1 << 28):
    """At every element, chunk by chunk on the device: the working weights are the
    master weights rounded to nearest even in their 16-bit format (torch's own
    conversion), v >= 0 (a sum of squares), and master, m, v finite."""
    n = master.numel()
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        rne = master[a:b].to(w16.dtype).view(torch.int16)
        assert torch.equal(rne, w16[a:b].view(torch.int16)), (what, "w16", a)
        assert bool((v[a:b] >= 0).all()), (what, "v", a)
        for k, t in (("master", master), ("m", m), ("v", v)):
            assert bool(torch.isfinite(t[a:b]).all()), (what, k, a)
    log(f"  {what}: w16 == RNE16(master), v >= 0, master/m/v finite at all {n} elements")


def every_element_vs_oracle(g16, before, after, dtype, t, S, hp, what, chunk=1 << 27):
    """One step of a full-size shard against the oracle at every element: chunk by
    chunk, the state before the step (device copies, or None for zeros) and the
    gradients go to pinned host buffers, the oracle steps them on the host's threads,
    and the device's result must meet the bar at every element."""
    n = g16.numel()
    c = min(chunk, n)
    pin = lambda dt: torch.empty(c, dtype=dt, pin_memory=True)
    hg, hw = pin(g16.dtype), pin(after["w16"].dtype)
    state = {k: pin(torch.float32) for k in ("master", "m", "v")}
    got = {k: pin(torch.float32) for k in ("master", "m", "v")}
    w16_ref = np.zeros(c, np.uint16)
    bits16 = lambda x: x.view(torch.int16).numpy().view(np.uint16)
    worst = {}
    t0 = time.time()
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        L = b - a
        if a and (a // chunk) % 8 == 0:
            log(f"  {what}: {a} of {n} elements compared ({time.time() - t0:.0f} s)")
        hg[:L].copy_(g16[a:b])
        hw[:L].copy_(after["w16"][a:b])
        for k in ("master", "m", "v"):
            if before[k] is None:
                state[k][:L].zero_()
            else:
                state[k][:L].copy_(before[k][a:b])
            got[k][:L].copy_(after[k][a:b])
        h = {k: state[k][:L].numpy() for k in ("master", "m", "v")}
        h["w16"] = w16_ref[:L]
        oracle.adam_step_mt(h["w16"], bits16(hg[:L]), h["master"], h["m"], h["v"], dtype, step=t,
                            loss_scale=S, **hp)
        dev = {k: got[k][:L].numpy() for k in ("master", "m", "v")}
        dev["w16"] = bits16(hw[:L])
        st = assert_close(dev, h, dtype, f"{what} [{a}, {b})")
        for k, (mx, nz) in st.items():
            pm, pn = worst.get(k, (0, 0))
            worst[k] = (max(pm, mx), pn + nz)
    log(f"  {what} step {t} at all {n} elements against the oracle ({time.time() - t0:.0f} s): "
        f"(max ulp, non-bitwise) {worst}")
    return worst


def take(t, wins, conv):
    return [conv(t[a:b]) for a, b in wins]


def run_windows_oracle(host, grads_per_step, dtype, hp, steps, S):
    for i in range(len(host)):
        h = host[i]
        for t, gw in zip(steps, grads_per_step):
            oracle.adam_step(h["w16"], gw[i], h["master"], h["m"], h["v"], dtype, step=t,
                             loss_scale=S, **hp)


def test_c3_bf16_warm_shard_windows():
    w = synth.WORKLOADS[3]
    psi, n, r = w.psi, w.n, w.ranks[0]
    lay = zs.zero_shard_layout(psi, n, r)
    cnt, hp, S = lay.count, hp_of(w), w.loss_scale
    assert cnt == 937_500_000
    log(f"C3 allocating 5 x {cnt} elements")
    g16 = torch.empty(cnt, dtype=torch.bfloat16, device=DEV)
    master = synth.fill_normal_(torch.empty(cnt, device=DEV), w.master_std, synth.seed_of(3, 2))
    m = torch.empty(cnt, device=DEV)
    v = torch.empty(cnt, device=DEV)
    synth.fill_warm_moments_(m, v, w.grad_std, synth.seed_of(3, 3), w.beta1, w.beta2,
                             w.warm_steps)
    w16 = torch.zeros(cnt, dtype=torch.bfloat16, device=DEV)
    wins = windows_of(cnt, np.random.default_rng(3))
    host = [dict(master=a, m=b, v=c, w16=np.zeros(a.size, np.uint16))
            for a, b, c in zip(take(master, wins, f32), take(m, wins, f32), take(v, wins, f32))]
    flag = flag_buf()
    steps = list(range(w.warm_steps + 1, w.warm_steps + w.steps + 1))
    gsteps = []
    for i, t in enumerate(steps):
        synth.fill_normal_(g16, w.grad_std, synth.seed_of(3, 1, i + 1))
        gsteps.append(take(g16, wins, u16))
        zs.zero_overflow_check(g16, psi, n, r, S, flag)
        if i in (0, len(steps) - 1):
            assert oracle.overflow_flag_mt(u16(g16), "bf16", S) == flag.item() == 0
        before = dict(master=master.clone(), m=m.clone(), v=v.clone()) if i == 0 else None
        zs.zero_adam_step(w16, g16, master, m, v, psi, n, r, step=t, loss_scale=S,
                          found_inf=flag, **hp)
        if i == 0:   # the first step (warm moments, t = 101) at every element
            torch.cuda.synchronize()
            every_element_vs_oracle(g16, before, dict(master=master, m=m, v=v, w16=w16), "bf16",
                                    t, S, hp, "C3")
            del before
            torch.cuda.empty_cache()
    torch.cuda.synchronize()
    log("C3 GPU steps done; oracle on windows")
    run_windows_oracle(host, gsteps, "bf16", hp, steps, S)
    got = [dict(master=a, m=b, v=c, w16=d) for a, b, c, d in
           zip(take(master, wins, f32), take(m, wins, f32), take(v, wins, f32),
               take(w16, wins, u16))]
    cat = lambda lst, k: np.concatenate([x[k] for x in lst])
    keys = ("master", "m", "v", "w16")
    log("  C3 windows", assert_close({k: cat(got, k) for k in keys},
                                     {k: cat(host, k) for k in keys}, "bf16", "C3"))
    full_buffer_invariants(master, m, v, w16, "C3")


def test_c4_ten_billion_unsharded_windows():
    w = synth.WORKLOADS[4]
    psi = w.psi
    hp, S = hp_of(w), w.loss_scale
    free, total = torch.cuda.mem_get_info(DEV)
    need = psi * 16 + (1 << 30)
    # a copy of the starting master for the every-element check of the first step
    full_check = free >= need + psi * 4
    if free < need:
        pytest.skip(f"needs {need / 1e9:.0f} GB of device memory, {free / 1e9:.0f} GB free")
    log(f"C4 allocating 160 GB ({free / 1e9:.0f} GB free)")
    g16 = synth.fill_normal_(torch.empty(psi, dtype=torch.float16, device=DEV), w.grad_std,
                             synth.seed_of(4, 1))
    master = synth.fill_normal_(torch.empty(psi, device=DEV), w.master_std, synth.seed_of(4, 2))
    m = torch.zeros(psi, device=DEV)
    v = torch.zeros(psi, device=DEV)
    w16 = torch.zeros(psi, dtype=torch.float16, device=DEV)
    wins = windows_of(psi, np.random.default_rng(4))
    assert wins[-1][1] == psi and any(a > 2 ** 32 for a, _ in wins)
    host = [dict(master=a, m=np.zeros(a.size, np.float32), v=np.zeros(a.size, np.float32),
                 w16=np.zeros(a.size, np.uint16)) for a in take(master, wins, f32)]
    gw = take(g16, wins, u16)
    flag = flag_buf()
    steps = list(range(1, w.steps + 1))
    master0 = master.clone() if full_check else None
    if not full_check:
        log(f"  C4: {free / 1e9:.0f} GB free, too little for the every-element check; windows only")
    for t in steps:
        zs.zero_overflow_check(g16, psi, 1, 0, S, flag)
        zs.zero_adam_step(w16, g16, master, m, v, psi, 1, 0, step=t, loss_scale=S,
                          found_inf=flag, **hp)
        log(f"  step {t} enqueued")
        if t == 1 and full_check:   # the first step at every element, as bench.py launches it
            torch.cuda.synchronize()
            assert flag.item() == 0
            every_element_vs_oracle(g16, dict(master=master0, m=None, v=None),
                                    dict(master=master, m=m, v=v, w16=w16), "f16", t, S, hp, "C4")
            del master0
            torch.cuda.empty_cache()
    torch.cuda.synchronize()
    assert flag.item() == 0
    run_windows_oracle(host, [gw] * len(steps), "f16", hp, steps, S)
    got = [dict(master=a, m=b, v=c, w16=d) for a, b, c, d in
           zip(take(master, wins, f32), take(m, wins, f32), take(v, wins, f32),
               take(w16, wins, u16))]
    cat = lambda lst, k: np.concatenate([x[k] for x in lst])
    keys = ("master", "m", "v", "w16")
    log("  C4 windows", assert_close({k: cat(got, k) for k in keys},
                                     {k: cat(host, k) for k in keys}, "f16", "C4"))
    full_buffer_invariants(master, m, v, w16, "C4")
    # flag property at full size: one NaN far past 2^32 is seen, and only while there
    far = psi - 12345
    keep = g16[far].clone()
    g16[far] = float("nan")
    zs.zero_overflow_check(g16, psi, 1, 0, S, flag)
    assert flag.item() == 1
    g16[far] = keep
    zs.zero_overflow_check(g16, psi, 1, 0, S, flag)
    assert flag.item() == 0


def test_c6_one_and_a_half_billion_unsharded_windows():
    # the pages' plain data-parallel example: 1.5e9 parameters, 16 B each on one rank
    w = synth.WORKLOADS[6]
    psi, hp, S = w.psi, hp_of(w), w.loss_scale
    lay = zs.zero_shard_layout(psi, 1, 0)
    assert lay.count == psi and lay.bytes_dp == 24_000_000_000
    log(f"C6 allocating 5 x {psi} elements (24 GB)")
    master = synth.fill_normal_(torch.empty(psi, device=DEV), w.master_std, synth.seed_of(6, 2))
    m = torch.zeros(psi, device=DEV)
    v = torch.zeros(psi, device=DEV)
    g16 = torch.empty(psi, dtype=torch.bfloat16, device=DEV)
    w16 = torch.zeros(psi, dtype=torch.bfloat16, device=DEV)
    wins = windows_of(psi, np.random.default_rng(6))
    assert wins[-1][1] == psi
    host = [dict(master=a, m=np.zeros(a.size, np.float32), v=np.zeros(a.size, np.float32),
                 w16=np.zeros(a.size, np.uint16)) for a in take(master, wins, f32)]
    flag = flag_buf()
    steps = list(range(1, w.steps + 1))
    gsteps = []
    for t in steps:
        synth.fill_normal_(g16, w.grad_std, synth.seed_of(6, 1, t))
        gsteps.append(take(g16, wins, u16))
        zs.zero_overflow_check(g16, psi, 1, 0, S, flag)
        last = t == steps[-1]
        before = dict(master=master.clone(), m=m.clone(), v=v.clone()) if last else None
        zs.zero_adam_step(w16, g16, master, m, v, psi, 1, 0, step=t, loss_scale=S,
                          found_inf=flag, **hp)
        if last:   # the last step (moments of nine steps, t = 10) at every element
            torch.cuda.synchronize()
            every_element_vs_oracle(g16, before, dict(master=master, m=m, v=v, w16=w16), "bf16",
                                    t, S, hp, "C6")
            del before
            torch.cuda.empty_cache()
    torch.cuda.synchronize()
    assert flag.item() == 0
    log("C6 GPU steps done; oracle on windows")
    run_windows_oracle(host, gsteps, "bf16", hp, steps, S)
    got = [dict(master=a, m=b, v=c, w16=d) for a, b, c, d in
           zip(take(master, wins, f32), take(m, wins, f32), take(v, wins, f32),
               take(w16, wins, u16))]
    cat = lambda lst, k: np.concatenate([x[k] for x in lst])
    keys = ("master", "m", "v", "w16")
    log("  C6 windows", assert_close({k: cat(got, k) for k in keys},
                                     {k: cat(host, k) for k in keys}, "bf16", "C6"))
    full_buffer_invariants(master, m, v, w16, "C6")


# ---------------------------------------------------------------------------
# C5: ragged last rank of 64, overflow injection, skip + loss-scale halving
# ---------------------------------------------------------------------------

def test_c5_ragged_rank63_overflow_schedule():
    w = synth.WORKLOADS[5]
    psi, n, r = w.psi, w.n, 63
    for rr in range(n):
        assert zs.zero_shard_layout(psi, n, rr).__dict__ == oracle.layout(psi, n, rr).__dict__
    lay = zs.zero_shard_layout(psi, n, r)
    cnt, pad, phase = lay.count, lay.pad, lay.offset % 8
    assert (cnt, pad, phase) == (137_656_190, 61, 5)
    hp = hp_of(w)
    # shard-local buffers that keep the rank's real alignment phase; the padding
    # of the 16-bit gradients holds NaN sentinels that must never be read
    V = {k: GuardedView(cnt + pad, torch.float16 if k in ("g16", "w16") else torch.float32,
                        phase, DEV) for k in ("g16", "w16", "master", "m", "v")}
    views = {k: gv.view[:cnt] for k, gv in V.items()}
    synth.fill_normal_(views["master"], w.master_std, synth.seed_of(5, 2))
    views["m"].zero_()
    views["v"].zero_()
    views["w16"].zero_()
    ref = host_state(f32(views["master"]), np.zeros(cnt, np.float32), np.zeros(cnt, np.float32),
                     np.zeros(cnt, np.uint16))
    other_rng = np.random.default_rng(synth.seed_of(5, 6))
    gpu_state = zs.Scaler(loss_scale=w.loss_scale)
    ref_state = oracle.ScalerState(loss_scale=w.loss_scale)
    flag = flag_buf()
    trace = []
    for step in range(1, w.steps + 1):
        synth.fill_normal_(views["g16"], w.grad_std, synth.seed_of(5, 1, step))
        injected = 0
        others = 0
        if step % 2 == 0:
            injected = synth.inject_nonfinite_(views["g16"], w.inject_prob,
                                               synth.seed_of(5, 5, step)).size
            assert injected > 0
            # the other 63 ranks, simulated on the host
            others = int(other_rng.binomial(psi - cnt, w.inject_prob))
        g_host = u16(views["g16"])
        S_gpu, S_ref = gpu_state.loss_scale, ref_state.loss_scale
        zs.zero_overflow_check(views["g16"], psi, n, r, S_gpu, flag)
        local = int(flag.item())
        ref_local = oracle.overflow_flag_mt(g_host, "f16", S_ref)
        assert local == ref_local, step
        apply_gpu = zs.zero_scaler_update(gpu_state, int(local or others > 0))
        apply_ref = oracle.policy(ref_state, ref_local or others > 0)
        assert apply_gpu == apply_ref
        assert (gpu_state.step, gpu_state.loss_scale) == (ref_state.step, ref_state.loss_scale)
        if apply_gpu:
            zs.zero_adam_step(views["w16"], views["g16"], views["master"], views["m"],
                              views["v"], psi, n, r, step=gpu_state.step, loss_scale=S_gpu,
                              **hp)
            oracle.adam_step_mt(ref["w16"], g_host, ref["master"], ref["m"], ref["v"], "f16",
                                step=ref_state.step, loss_scale=S_ref, **hp)
        trace.append((step, injected, local, apply_gpu, gpu_state.step, gpu_state.loss_scale))
        log(f"  C5 step {step}: injected {injected} local flag {local} applied {apply_gpu} "
            f"t={gpu_state.step} S={gpu_state.loss_scale}")
    torch.cuda.synchronize()
    assert gpu_state.step == 5 and gpu_state.loss_scale == 2048.0
    assert [a for *_, a, _, _ in trace] == [True, False] * 5
    got = {k: (f32 if k in ("master", "m", "v") else u16)(views[k]) for k in ref}
    log("  C5 vs oracle", assert_close(got, ref, "f16", "C5"))
    # padding and guards untouched (the g16 padding still holds its NaN sentinels)
    for k, gv in V.items():
        tail = (u16 if k in ("g16", "w16") else f32)(gv.view[cnt:])
        if k in ("g16", "w16"):
            assert np.all(tail == SENT16), k
        else:
            assert np.all(tail.view(np.uint32) == 0x7FC0DEAD), k
        assert gv.guards_intact(), k
