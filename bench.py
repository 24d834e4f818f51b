#!/usr/bin/env python3
"""Benchmark of the ZeRO-sharded mixed-precision Adam step on one MI355X.

A step is one pass of the whole hot path over the shard:
  layout (host) -> unscale + overflow check (GPU, 2 B/param) -> 4-byte flag
  read back -> skip-or-apply decision and loss scale (host) -> Adam step (GPU,
  28 B/param, writes the 16-bit working copy).
Inputs are synthetic, seeded and resident in HBM before the timed region.

Default workload: 1e10 parameters, N = 1 (the 160 GB unsharded case), FP16
gradients ~N(0,1e-3) carrying a loss scale of 65536, FP32 master ~N(0,0.02),
m = v = 0 at the start, AdamW lr 1e-4, wd 0.1.

Prints one JSON line: params/s over the timed steps, the step kernel's HBM
roofline (algorithmic 28 B/param over its HIP-event-timed duration, against the
8 TB/s peak; the library enqueues a step as consecutive launches of the step
kernel, so this is the launches' average bytes over their average duration with
the gaps between them counted), the HBM traffic per step measured by rocprofv3
counters when the profiled kernel's machine code matches the built one, the parity of the
run's own steps against the oracle (windows of the benchmarked buffers
replayed on the host, and the flag of every step against the oracle's over the
whole gradient buffer), the same measurements on the other roofline
configurations (the 7.5B rank, the ragged 8.81B rank, 1.5B) under
'workloads', and the CPU oracle timed on a bounded sample of the same inputs.

    python bench.py [--gpus 1] [--steps 5] [--warmup 2] [--workload 4]
"""
import argparse
import importlib.util
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "shard Adam params/sec + achieved HBM GB/s (28 B/param) vs peak, 1×MI355X"
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E, published
STEP_BYTES_PER_PARAM = 28       # read g 2 + master/m/v 12; write master/m/v 12 + w16 2
CHECK_BYTES_PER_PARAM = 2
BUILD_SCRIPT = os.path.join(ROOT, "zero_sharded_mixed_shard_amd", "build.py")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "adam_step_flat10B_hbm_traffic.md")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def built_isa_hashes() -> dict:
    """Per-kernel machine-code hashes that the build wrote beside the library."""
    spec = importlib.util.spec_from_file_location("zs_build", BUILD_SCRIPT)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.read_isa_hashes()


def traffic_profile(workload_name: str):
    """The machine-readable fields of the committed rocprofv3 counter summary, or None
    unless it was taken on this workload with the same machine code of the step kernel
    as the library built now."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                kv[k.strip()] = v.strip().strip("`")
    symbol = kv.get("kernel_symbol")
    if symbol is None or kv.get("kernel_isa_sha256") != built_isa_hashes().get(symbol):
        return None
    if kv.get("workload") != workload_name:
        return None
    return kv


def measured_traffic(workload_name: str):
    """HBM bytes per step (the sum over its launches of the step kernel) from the committed
    rocprofv3 counter summary, or None (see traffic_profile)."""
    kv = traffic_profile(workload_name)
    try:
        return float(kv["hbm_bytes_per_step"]) if kv else None
    except (KeyError, ValueError):
        return None


def launches_per_step(workload_name: str):
    """Launches of the step kernel per step, as the same summary's trace counted them
    (the library enqueues a long shard's step as consecutive launches), or None."""
    kv = traffic_profile(workload_name)
    try:
        return int(kv["launches_per_step"]) if kv else None
    except (KeyError, ValueError):
        return None


def make_workload(cfg: int, dev):
    import torch

    import synth
    import zero_sharded_mixed_shard_amd as zs

    w = synth.WORKLOADS[cfg]
    rank = w.ranks[-1]
    lay = zs.zero_shard_layout(w.psi, w.n, rank)
    cnt = lay.count
    # shard-local buffers that keep the rank's alignment phase in the flat buffer
    phase = lay.offset % 8
    td = w.torch_dtype

    def alloc(dtype):
        return torch.empty(phase + cnt, dtype=dtype, device=dev)[phase:]

    t0 = time.time()
    # FP32 state first, then the 16-bit arrays: on MI355X this allocation order
    # measured a 1-2% faster step at 160 GB than allocating the 16-bit arrays
    # first (where the driver places the arrays changes the streaming rate).
    bufs = dict(master=alloc(torch.float32), m=alloc(torch.float32), v=alloc(torch.float32))
    bufs.update(g16=alloc(td), w16=alloc(td))
    synth.fill_normal_(bufs["g16"], w.grad_std, synth.seed_of(cfg, 1))
    synth.fill_normal_(bufs["master"], w.master_std, synth.seed_of(cfg, 2))
    if w.warm_steps:
        synth.fill_warm_moments_(bufs["m"], bufs["v"], w.grad_std, synth.seed_of(cfg, 3),
                                 w.beta1, w.beta2, w.warm_steps)
    else:
        bufs["m"].zero_()
        bufs["v"].zero_()
    bufs["w16"].zero_()
    torch.cuda.synchronize()
    log(f"[bench] {w.name}: rank {rank}/{w.n}, {cnt} params, inputs ready in "
        f"{time.time() - t0:.1f}s")
    return w, rank, lay, bufs


PARITY_WINDOW = 8192
PARITY_RANDOM = 8


def parity_windows(count: int, seed: int) -> list:
    """Element ranges whose state the oracle replays: head, tail, past 2^32, and seeded
    random windows of PARITY_WINDOW elements."""
    import numpy as np

    w = min(PARITY_WINDOW, count)
    starts = {0, count - w}
    if count > (1 << 32) + w:
        starts.add(1 << 32)
    rng = np.random.default_rng(seed)
    for _ in range(PARITY_RANDOM):
        starts.add(int(rng.integers(0, count - w + 1)))
    return sorted((a, a + w) for a in starts)


def snapshot(bufs, wins) -> list:
    """Host copies of every buffer over each window (16-bit arrays as bit patterns)."""
    import synth

    out = []
    for a, b in wins:
        out.append({k: (synth.to_numpy_u16(bufs[k][a:b]) if k in ("g16", "w16")
                        else bufs[k][a:b].cpu().numpy().copy())
                    for k in ("g16", "master", "m", "v", "w16")})
    return out


def full_flag_oracle(g16, dtype: str, loss_scale: float, chunk: int = 1 << 28) -> int:
    """The oracle's overflow flag over a whole device gradient buffer, in host chunks."""
    import oracle
    import synth

    n = g16.numel()
    for a in range(0, n, chunk):
        if oracle.overflow_flag_mt(synth.to_numpy_u16(g16[a:min(n, a + chunk)]), dtype,
                                   loss_scale):
            return 1
    return 0


def replay_parity(w, start, final, applied, flags) -> dict:
    """Replay the run's applied steps (t, S) through the oracle on the start windows and
    compare with the device's final windows: max ulp and non-bitwise counts per array,
    and the device's flag of every step against the oracle's over the whole buffer."""
    import numpy as np

    import oracle

    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay)
    stats = {k: [0, 0] for k in ("master", "m", "v", "w16")}
    elems = 0
    for s0, s1 in zip(start, final):
        ref = {k: s0[k].copy() for k in ("master", "m", "v", "w16")}
        for t, S in applied:
            oracle.adam_step(ref["w16"], s0["g16"], ref["master"], ref["m"], ref["v"], w.dtype,
                             step=t, loss_scale=S, **hp)
        elems += s0["g16"].size
        for k in ("master", "m", "v"):
            d = oracle.ulp_distance32(s1[k], ref[k])
            stats[k][0] = max(stats[k][0], int(d.max()))
            stats[k][1] += int(np.count_nonzero(s1[k].view(np.uint32) != ref[k].view(np.uint32)))
        d = oracle.ulp_distance16(s1["w16"], ref["w16"], w.dtype)
        stats["w16"][0] = max(stats["w16"][0], int(d.max()))
        stats["w16"][1] += int(np.count_nonzero(s1["w16"] != ref["w16"]))
    flags_equal = all(got == want for got, want in flags)
    return {"windows": len(start), "elements": elems, "steps_replayed": len(applied),
            "max_ulp": {k: v[0] for k, v in stats.items()},
            "non_bitwise": {k: v[1] for k, v in stats.items()},
            "flag_steps": len(flags), "flags_equal": flags_equal,
            "bar": "master/m/v <= 2 ulp, w16 <= 1 ulp, flag bit-exact",
            "ok": flags_equal and all(stats[k][0] <= 2 for k in ("master", "m", "v"))
            and stats["w16"][0] <= 1}


def layouts_equal(psi: int, n: int) -> bool:
    """Every rank's layout from the library equals the oracle's, field by field."""
    import oracle
    import zero_sharded_mixed_shard_amd as zs

    return all(zs.zero_shard_layout(psi, n, r).__dict__ == oracle.layout(psi, n, r).__dict__
               for r in range(n))


def run_steps(w, rank, lay, b, dev, warmup: int, steps: int, stream, seed: int) -> dict:
    """The host-controlled sequence (check, 4-byte read-back, decision, step) on one
    workload's buffers: HIP-event times of the check and the step over the timed steps,
    and the parity of every step against the oracle."""
    import torch

    import zero_sharded_mixed_shard_amd as zs

    psi, n, cnt = w.psi, w.n, lay.count
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    scaler = zs.Scaler(w.loss_scale, step=w.warm_steps)
    wins = parity_windows(cnt, seed)
    start = snapshot(b, wins)
    applied, found_flags, ev = [], [], []
    for i in range(warmup + steps):
        timed = i >= warmup
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if timed else None
        S = scaler.loss_scale
        if timed:
            e[0].record(stream)
        zs.zero_overflow_check(b["g16"], psi, n, rank, S, flag, stream=stream)
        if timed:
            e[1].record(stream)
        found = int(flag.item())
        found_flags.append((found, S))
        if zs.zero_scaler_update(scaler, found):
            if timed:
                e[2].record(stream)
            zs.zero_adam_step(b["w16"], b["g16"], b["master"], b["m"], b["v"], psi, n, rank,
                              step=scaler.step, loss_scale=S, found_inf=flag, stream=stream, **hp)
            applied.append((scaler.step, S))
            if timed:
                e[3].record(stream)
                ev.append(e)
    torch.cuda.synchronize()
    final = snapshot(b, wins)
    want = {S: full_flag_oracle(b["g16"], w.dtype, S) for S in {S for _, S in found_flags}}
    parity = replay_parity(w, start, final, applied, [(f, want[S]) for f, S in found_flags])
    parity["layouts_equal"] = layouts_equal(w.psi, w.n)
    parity["ok"] = parity["ok"] and parity["layouts_equal"]
    step_ms = [x[2].elapsed_time(x[3]) for x in ev]
    check_ms = [x[0].elapsed_time(x[1]) for x in ev]
    return {"step_ms": step_ms, "check_ms": check_ms, "parity": parity}


def measure_workloads(dev, ids, warmup: int, steps: int) -> dict:
    """The other roofline configurations, one after another: the check and the step timed
    with HIP events (median and min) and the parity of the run's steps."""
    import statistics

    import torch

    out = {}
    for cfg in ids:
        w, rank, lay, b = make_workload(cfg, dev)
        stream = torch.cuda.current_stream(dev)
        r = run_steps(w, rank, lay, b, dev, warmup, steps, stream, seed=cfg)
        cnt = lay.count
        med, mn = statistics.median(r["step_ms"]), min(r["step_ms"])
        cmed = statistics.median(r["check_ms"])
        gbps = STEP_BYTES_PER_PARAM * cnt / (med * 1e-3) / 1e9
        out[w.name] = {
            "shard_params": cnt, "psi": w.psi, "zero_ranks": w.n, "rank": rank,
            "grad_weight_dtype": w.dtype, "steps": steps, "warmup": warmup,
            "adam_step_ms_median": med, "adam_step_ms_min": mn,
            "adam_step_GBps": gbps, "frac": gbps / PEAK_HBM_GBPS,
            "adam_step_params_per_s": cnt / (med * 1e-3),
            "overflow_check_ms_median": cmed, "overflow_check_ms_min": min(r["check_ms"]),
            "overflow_check_GBps": CHECK_BYTES_PER_PARAM * cnt / (cmed * 1e-3) / 1e9,
            "parity": r["parity"]}
        log(f"[bench] {w.name}: step {med:.4f} ms ({gbps / 1e3:.3f} TB/s), parity "
            f"{'ok' if r['parity']['ok'] else 'FAILED'}")
        del b
        torch.cuda.empty_cache()
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(bufs, w, budget_s: float, sample: int):
    """The oracle as it stands, on the host's cores, over a slice of the same inputs.

    A quarter of the budget times it on one thread, the rest on the host's CPU
    share (the threads this process may use: 16 on the MI355X machines, whatever
    the machine's core count); the reported value is the latter."""
    import numpy as np

    import oracle
    import synth

    n = min(sample, bufs["g16"].numel())
    g = synth.to_numpy_u16(bufs["g16"][:n])
    master0 = bufs["master"][:n].cpu().numpy().copy()
    m0 = bufs["m"][:n].cpu().numpy().copy()
    v0 = bufs["v"][:n].cpu().numpy().copy()
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay)

    def run(threads, seconds):
        master, m, v = master0.copy(), m0.copy(), v0.copy()
        w16 = np.zeros(n, np.uint16)
        steps, t0 = 0, time.perf_counter()
        while True:
            used = oracle.adam_step_mt(w16, g, master, m, v, w.dtype, threads=threads,
                                       step=steps + 1, loss_scale=w.loss_scale, **hp)
            steps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                return n * steps / el, used, steps, el

    one, _, steps1, el1 = run(1, budget_s / 4)
    share = oracle.host_threads()
    rate, used, steps, el = run(share, budget_s * 3 / 4)
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = None
    return {"value": rate, "unit": "params/s", "cores": used, "kind": "oracle",
            "sample": f"first {n} params of the same shard inputs, {steps} Adam steps "
                      f"({el:.1f} s wall) on {used} host threads",
            "threads_used": used, "nproc": os.cpu_count(), "affinity_cpus": affinity,
            "threads_rule": "the host's CPU share: at most 16 threads (the worker budget per "
                            "GPU on the MI355X machines), fewer if the affinity mask is smaller",
            "single_thread": {"value": one, "unit": "params/s",
                              "sample": f"same slice, {steps1} Adam steps ({el1:.1f} s wall)"},
            "GBps": rate * STEP_BYTES_PER_PARAM / 1e9, "cpu": cpu_model()}


def copy_bandwidth(dev, gib: int = 4):
    """Same-run plain device copies of gib GiB, GB/s of read + write bytes: the
    runtime's copy (torch copy_), and the library's own streaming copy (a one-shard
    all-gather: one read and one write stream with the step's 16-B, one-tile-per-block
    access pattern)."""
    import torch

    import zero_sharded_mixed_shard_amd as zs

    n = gib * (1 << 30) // 4
    a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    reps = 5

    def rate(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return 2 * n * 4 / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9

    runtime = rate(lambda: b.copy_(a))
    stream = rate(lambda: zs.zero_gather_shards(b, [a], n, 1))
    del a, b
    torch.cuda.empty_cache()
    return runtime, stream


def measure_extras(dev, n_elem: int = 1 << 30, reps: int = 5) -> dict:
    """Bandwidth of the path's other kernels on n_elem-element shards (HIP events).

    Algorithmic bytes per element: accumulate 10 (read 2 + 4, write 4), FP32
    check 4, accumulate with the FP32 check fused 10, 16-bit check with the sum
    of squares 2 (S a power of two, and S = 3),
    FP32-gradient step 30, reduce of 8 FP16 replicas into FP16 18 (read
    8 x 2, write 2), the same reduce with the check of its chunk fused in 18,
    the 16-bit check of that chunk alone 2, gather of 8 FP16 shards 4 (read 2,
    write 2), and the device-controlled check + decision + step 30 (2 + 28)."""
    import torch

    import synth
    import zero_sharded_mixed_shard_amd as zs

    out = {}
    stream = torch.cuda.current_stream(dev)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def record(name, ms, elems, bpe):
        gbps = bpe * elems / (ms * 1e-3) / 1e9
        out[name] = {"ms": ms, "elements": elems, "bytes_per_elem": bpe, "GBps": gbps,
                     "frac": gbps / PEAK_HBM_GBPS}

    n = n_elem
    hp = dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)
    g16 = synth.fill_normal_(torch.empty(n, dtype=torch.float16, device=dev), 1e-3, 1)
    acc = torch.zeros(n, device=dev)
    zs.zero_grad_accumulate(acc, g16, n, 1, 0, first=True)
    record("grad_accumulate", timed(lambda: zs.zero_grad_accumulate(acc, g16, n, 1, 0,
                                                                    first=False)), n, 10)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    record("overflow_check_g32", timed(lambda: zs.zero_overflow_check_g32(acc, n, 1, 0, 65536.0,
                                                                          flag)), n, 4)
    # the last micro-batch with the FP32 check fused in: the accumulate's 10 B
    # per element, in place of 10 + 4 for the accumulate followed by the check
    record("grad_accumulate_check", timed(lambda: zs.zero_grad_accumulate_check(
        acc, g16, n, 1, 0, first=False, loss_scale=65536.0, found_inf=flag)), n, 10)
    sumsq = torch.zeros(1, device=dev)
    parts = torch.empty(zs.SUMSQ_PARTIALS, dtype=torch.float64, device=dev)
    record("overflow_check_sumsq_f16", timed(lambda: zs.zero_overflow_check(
        g16, n, 1, 0, 65536.0, flag, sumsq, parts)), n, 2)
    record("overflow_check_sumsq_f16_S3", timed(lambda: zs.zero_overflow_check(
        g16, n, 1, 0, 3.0, flag, sumsq, parts)), n, 2)
    master = synth.fill_normal_(torch.empty(n, device=dev), 0.02, 2)
    m = torch.zeros(n, device=dev)
    v = torch.zeros(n, device=dev)
    w16 = torch.zeros(n, dtype=torch.float16, device=dev)
    record("adam_step_g32", timed(lambda: zs.zero_adam_step_g32(
        w16, acc, master, m, v, n, 1, 0, step=1, loss_scale=65536.0 * 8, **hp)), n, 30)
    ctl = zs.device_ctl_new(65536.0, dev)
    bias = zs.zero_bias_corrections(0.9, 0.999, 1, 64).to(dev)

    def dev_step():
        zs.zero_overflow_check_dev(g16, n, 1, 0, ctl)
        zs.zero_scaler_update_dev(ctl, bias, 1)
        zs.zero_adam_step_dev(w16, g16, master, m, v, n, 1, 0, ctl=ctl, **hp)

    record("device_controlled_step", timed(dev_step), n, 30)
    del acc, m, v, master, ctl
    torch.cuda.empty_cache()
    # exchanges: 8 ranks, flat buffer of n elements
    ranks = 8
    reps16 = [synth.fill_normal_(torch.empty(n, dtype=torch.float16, device=dev), 1e-2, 10 + k)
              for k in range(ranks)]
    lay = zs.zero_shard_layout(n, ranks, 0)
    shard = torch.empty(lay.count, dtype=torch.float16, device=dev)
    record("reduce_shard_8x_f16", timed(lambda: zs.zero_reduce_shard(shard, reps16, n, ranks, 0)),
           lay.count, 2 * ranks + 2)
    # the reduce with the overflow check of its chunk fused in: the reduce's 18 B per
    # chunk element, in place of 18 + 2 for the reduce followed by the 16-bit check
    record("reduce_shard_check_8x_f16", timed(lambda: zs.zero_reduce_shard_check(
        shard, reps16, n, ranks, 0, 65536.0, flag)), lay.count, 2 * ranks + 2)
    record("overflow_check_f16_chunk", timed(lambda: zs.zero_overflow_check(
        shard, lay.count, 1, 0, 65536.0, flag)), lay.count, 2)
    shards = [r[:zs.zero_shard_layout(n, ranks, k).count].clone() for k, r in enumerate(reps16)]
    del reps16
    record("gather_shards_8x_f16", timed(lambda: zs.zero_gather_shards(w16, shards, n, ranks)),
           n, 4)
    return out


def measure_small(dev, steps: int = 300, warmup: int = 20) -> dict:
    """Whole-step time of the launch-bound workloads under three kinds of control.

    For each small workload (the 1M-parameter rank and one GPT-2-small rank):
    host control (the flag read back every step, as the main loop does),
    device control (check, decision and step enqueued with no read-back), and
    the device-controlled step captured once into a HIP graph and replayed.
    Times are wall-clock per step over `steps` steps between synchronisations."""
    import torch

    import zero_sharded_mixed_shard_amd as zs

    out = {}
    for cfg in (1, 2):
        w, rank, lay, b = make_workload(cfg, dev)
        psi, n, cnt = w.psi, w.n, lay.count
        hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                  weight_decay=w.weight_decay)
        flag = torch.zeros(1, dtype=torch.int32, device=dev)
        scaler = zs.Scaler(w.loss_scale)
        total = 3 * (warmup + steps) + 8
        ctl = zs.device_ctl_new(w.loss_scale, dev)
        bias = zs.zero_bias_corrections(w.beta1, w.beta2, 1, total).to(dev)

        def host_step():
            zs.zero_overflow_check(b["g16"], psi, n, rank, scaler.loss_scale, flag)
            S = scaler.loss_scale
            if zs.zero_scaler_update(scaler, int(flag.item())):
                zs.zero_adam_step(b["w16"], b["g16"], b["master"], b["m"], b["v"], psi, n,
                                  rank, step=scaler.step, loss_scale=S, found_inf=flag, **hp)

        def device_step():
            zs.zero_overflow_check_dev(b["g16"], psi, n, rank, ctl)
            zs.zero_scaler_update_dev(ctl, bias, 1)
            zs.zero_adam_step_dev(b["w16"], b["g16"], b["master"], b["m"], b["v"], psi, n,
                                  rank, ctl=ctl, **hp)

        def per_step_ms(fn):
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                fn()
            torch.cuda.synchronize()
            return (time.perf_counter() - t0) / steps * 1e3

        res = {"shard_params": cnt, "host_control_ms": per_step_ms(host_step),
               "device_control_ms": per_step_ms(device_step)}
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            device_step()
        res["graph_replay_ms"] = per_step_ms(graph.replay)
        c = zs.device_ctl_read(ctl)
        if c.status != 0 or c.scaler.step != 2 * (warmup + steps):
            raise RuntimeError(f"device-controlled steps skipped: status {c.status}, "
                               f"t {c.scaler.step}")
        for k in ("host_control_ms", "device_control_ms", "graph_replay_ms"):
            res[k.replace("_ms", "_params_per_s")] = cnt / (res[k] * 1e-3)
        out[w.name] = res
        del graph, b
        torch.cuda.empty_cache()
    return out


def measure_checkpoint(n_elem: int = 1 << 26) -> dict:
    """Host throughput of the sharded checkpoint calls on two ranks' shards.

    psi = 2 * n_elem over N = 2: each rank's file holds n_elem elements (14 B
    each plus a 128-B header).  Timed, each twice (first and repeat): writing
    both files (temporary file, fsync, rename), verifying both payload hashes,
    reading one shard back, and reading rank 1 of a 3-rank layout from the two
    files.  Beside them, the same bytes written with numpy's tofile plus fsync
    and read back with fromfile: the file system's practical rate."""
    import tempfile

    import numpy as np

    import zero_sharded_mixed_shard_amd as zs

    n_old, n_new = 2, 3
    psi = n_old * n_elem
    rng = np.random.default_rng(7)
    shards = [(rng.integers(0, 1 << 16, n_elem, dtype=np.uint16),
               rng.standard_normal(n_elem, dtype=np.float32),
               rng.standard_normal(n_elem, dtype=np.float32),
               rng.random(n_elem, dtype=np.float32)) for _ in range(n_old)]
    file_bytes = 14 * n_elem + 128
    out = {"elements_per_shard": n_elem, "file_bytes": file_bytes}

    def timed(key, nbytes, fn):
        """Run fn twice; the first call after a write can wait on the file system."""
        rates = []
        for _ in range(2):
            t0 = time.perf_counter()
            fn()
            rates.append(nbytes / (time.perf_counter() - t0) / 1e9)
        out[key + "_GBps"] = rates[0]
        out[key + "_repeat_GBps"] = rates[1]

    def write_plain(path):
        with open(path, "wb") as f:
            for r in range(n_old):
                for a in shards[r]:
                    a.tofile(f)
            f.flush()
            os.fsync(f.fileno())

    def read_plain(path):
        with open(path, "rb") as f:
            for dt in (np.uint16, np.float32, np.float32, np.float32):
                np.fromfile(f, dtype=dt, count=n_elem)

    with tempfile.TemporaryDirectory(dir=os.environ.get("TMPDIR")) as d:
        paths = [os.path.join(d, f"rank{r}.zshard") for r in range(n_old)]
        timed("write", n_old * file_bytes, lambda: [
            zs.zero_ckpt_write(paths[r], psi, n_old, r, "f16", zs.Scaler(65536.0, step=10),
                               *shards[r]) for r in range(n_old)])
        timed("verify", n_old * file_bytes, lambda: [zs.zero_ckpt_verify(p) for p in paths])
        timed("read", 14 * n_elem, lambda: zs.zero_ckpt_read(paths[0], 0, n_elem))
        back = zs.zero_ckpt_read(paths[0], 0, n_elem)
        if not all(np.array_equal(a.view(np.uint8), b.view(np.uint8))
                   for a, b in zip(back, shards[0])):
            raise RuntimeError("checkpoint read-back differs from what was written")
        del back
        cnt_new = zs.zero_shard_layout(psi, n_new, 1).count
        timed("read_resharded", 14 * cnt_new,
              lambda: zs.zero_ckpt_read_resharded(paths, psi, n_new, 1))
        plain = os.path.join(d, "plain.bin")
        timed("plain_write", n_old * 14 * n_elem, lambda: write_plain(plain))
        timed("plain_read", 14 * n_elem, lambda: read_plain(plain))
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1,
                    help="GPUs (only 1: the step runs on one rank's shard)")
    ap.add_argument("--steps", type=int, default=5, help="timed steps")
    ap.add_argument("--warmup", type=int, default=2, help="untimed steps before them")
    ap.add_argument("--workload", type=int, default=4, choices=[1, 2, 3, 4, 5, 6],
                    help="workload id (4 = 1e10 params, N=1; the reported configuration)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-clock budget of the CPU oracle baseline")
    ap.add_argument("--cpu-sample", type=int, default=1 << 27,
                    help="parameters in the CPU baseline's sample")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU oracle baseline")
    ap.add_argument("--no-copy", action="store_true", help="skip the device-copy measurement")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the other roofline configurations (7.5B rank, ragged 8.81B "
                         "rank, 1.5B) reported under 'workloads'")
    ap.add_argument("--workload-steps", type=int, default=10,
                    help="timed steps of each configuration under 'workloads'")
    ap.add_argument("--extras", action="store_true",
                    help="also time the accumulate / FP32-gradient / device-control / exchange "
                         "kernels on shards of --extras-elems elements (reported under 'extras')")
    ap.add_argument("--extras-elems", type=int, default=1 << 30,
                    help="shard size of the --extras measurements (elements)")
    ap.add_argument("--small", action="store_true",
                    help="also time whole steps of the launch-bound small workloads under host "
                         "control, device control and HIP-graph replay (reported under 'small')")
    ap.add_argument("--ckpt", action="store_true",
                    help="also time the sharded checkpoint calls on two 2^26-element shard "
                         "files (reported under 'checkpoint')")
    ap.add_argument("--control", choices=["host", "device"], default="host",
                    help="skip-or-apply decision on the host (4-byte read-back per step) or in "
                         "device memory (no read-back)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: the step runs on one rank's shard and no multi-GPU "
              f"run is provided (asked for --gpus {args.gpus}, WORLD_SIZE {world}).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import zero_sharded_mixed_shard_amd as zs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w, rank, lay, b = make_workload(args.workload, dev)
    psi, n, cnt = w.psi, w.n, lay.count
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    scaler = zs.Scaler(w.loss_scale)
    if w.warm_steps:
        scaler.step = w.warm_steps
    stream = torch.cuda.current_stream(dev)
    ev = []
    applied, found_flags = [], []     # (t, S) of every applied update; (flag, S) of every check

    def one_step(timed: bool):
        layout = zs.zero_shard_layout(psi, n, rank)                          # shard range
        S = scaler.loss_scale
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if timed else None
        if timed:
            e[0].record(stream)
        zs.zero_overflow_check(b["g16"], psi, n, rank, S, flag, stream=stream)   # unscale + check
        if timed:
            e[1].record(stream)
        found = int(flag.item())                                            # 4 bytes to host
        found_flags.append((found, S))
        if zs.zero_scaler_update(scaler, found):                            # skip or apply
            if timed:
                e[2].record(stream)
            zs.zero_adam_step(b["w16"], b["g16"], b["master"], b["m"], b["v"], psi, n, rank,
                              step=scaler.step, loss_scale=S, found_inf=flag, stream=stream,
                              **hp)
            applied.append((scaler.step, S))
            if timed:
                e[3].record(stream)
                ev.append(e)
        return layout

    if args.control == "device":
        ctl = zs.device_ctl_new(w.loss_scale, dev, step=scaler.step)
        t_first = scaler.step + 1
        bias = zs.zero_bias_corrections(w.beta1, w.beta2, t_first,
                                        args.warmup + args.steps + 1).to(dev)

        def one_step(timed: bool):   # noqa: F811  (device-resident control)
            layout = zs.zero_shard_layout(psi, n, rank)
            e = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if timed else None
            if timed:
                e[0].record(stream)
            zs.zero_overflow_check_dev(b["g16"], psi, n, rank, ctl, stream=stream)
            if timed:
                e[1].record(stream)
            zs.zero_scaler_update_dev(ctl, bias, t_first, stream=stream)
            if timed:
                e[2].record(stream)
            zs.zero_adam_step_dev(b["w16"], b["g16"], b["master"], b["m"], b["v"], psi, n, rank,
                                  ctl=ctl, stream=stream, **hp)
            if timed:
                e[3].record(stream)
                ev.append(e)
            return layout

    wins = parity_windows(cnt, seed=args.workload)
    start = snapshot(b, wins)
    for _ in range(args.warmup):
        one_step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        one_step(True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    if args.control == "device":
        c = zs.device_ctl_read(ctl)
        total = args.warmup + args.steps
        if c.status != 0 or c.scaler.step != scaler.step + total:
            raise RuntimeError(f"device control skipped steps: status {c.status}, "
                               f"t {c.scaler.step}")
        applied = [(t_first + i, w.loss_scale) for i in range(total)]
        found_flags = [(c.found_inf, w.loss_scale)]
    step_ms = [x[2].elapsed_time(x[3]) for x in ev]
    check_ms = [x[0].elapsed_time(x[1]) for x in ev]
    if not step_ms:
        raise RuntimeError("every timed step overflowed; nothing was measured")
    avg_step_ms = sum(step_ms) / len(step_ms)
    avg_check_ms = sum(check_ms) / len(check_ms)
    achieved = STEP_BYTES_PER_PARAM * cnt / (avg_step_ms * 1e-3) / 1e9
    traffic = measured_traffic(w.name)
    launches = launches_per_step(w.name)

    log("[bench] parity of the run's steps against the oracle ...")
    final = snapshot(b, wins)
    want = {S: full_flag_oracle(b["g16"], w.dtype, S) for S in {S for _, S in found_flags}}
    parity = replay_parity(w, start, final, applied, [(f, want[S]) for f, S in found_flags])
    parity["layouts_equal"] = layouts_equal(psi, n)
    parity["ok"] = parity["ok"] and parity["layouts_equal"]
    log(f"[bench] parity {'ok' if parity['ok'] else 'FAILED'}: max ulp {parity['max_ulp']}")

    copy_gbps, stream_copy_gbps = (None, None) if args.no_copy else copy_bandwidth(dev)
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline ...")
        cpu = cpu_baseline(b, w, args.cpu_seconds, args.cpu_sample)
    del b
    torch.cuda.empty_cache()
    workloads = None
    if not args.no_workloads:
        log("[bench] other roofline configurations ...")
        workloads = measure_workloads(dev, [c for c in (3, 5, 6) if c != args.workload],
                                      warmup=2, steps=args.workload_steps)
    ckpt = None
    if args.ckpt:
        log("[bench] checkpoint files ...")
        ckpt = measure_checkpoint()
    small = None
    if args.small:
        log("[bench] small workloads ...")
        small = measure_small(dev)
    extras = None
    if args.extras:
        log("[bench] extras ...")
        extras = measure_extras(dev, n_elem=args.extras_elems)

    out = {
        "metric": METRIC,
        "value": cnt * args.steps / elapsed,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "psi": psi, "zero_ranks": n, "rank": rank,
                   "shard_params": cnt, "grad_weight_dtype": w.dtype,
                   "optimizer": "AdamW" if w.weight_decay else "Adam",
                   "loss_scale": w.loss_scale, "bytes_per_param": STEP_BYTES_PER_PARAM,
                   "control": args.control},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS,
                     "traffic": traffic,
                     # one step is this many launches of the step kernel (from the profile's
                     # trace); achieved = their average bytes over their average duration
                     "launches_per_step": launches,
                     "ms_per_launch": avg_step_ms / launches if launches else None},
        "kernels": {"adam_step_ms": avg_step_ms, "adam_step_ms_min": min(step_ms),
                    "adam_step_ms_median": statistics.median(step_ms),
                    "overflow_check_ms": avg_check_ms,
                    "overflow_check_ms_median": statistics.median(check_ms),
                    "overflow_check_GBps": CHECK_BYTES_PER_PARAM * cnt / (avg_check_ms * 1e-3)
                    / 1e9,
                    "device_copy_GBps": copy_gbps,
                    "stream_copy_GBps": stream_copy_gbps,
                    # the step's algorithmic rate as a fraction of the library's own plain
                    # streaming copy in this run: the practical ceiling of a stream that
                    # mixes reads and writes
                    "step_vs_stream_copy": (achieved / stream_copy_gbps
                                            if stream_copy_gbps else None)},
        "parity": parity,
        "cpu_baseline": cpu,
    }
    if workloads is not None:
        out["workloads"] = workloads
    if extras is not None:
        out["extras"] = extras
    if small is not None:
        out["small"] = small
    if ckpt is not None:
        out["checkpoint"] = ckpt
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
