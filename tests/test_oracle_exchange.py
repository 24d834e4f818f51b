"""Pins for the oracle's exchange stand-ins (reduce-scatter, all-gather) and
its communication / peak-memory accounting.

* reduce-scatter followed by all-gather equals the all-reduce (the element-wise
  sum of the full replicas) -- the identity the pages build ZeRO on ("Training
  models too big for one GPU", "Data parallelism and the all-reduce");
* sums of identical or integer replicas are exact; FP32 sums stay within the
  recursive-summation bound of math.fsum;
* all-gather puts every element of every shard at its flat index (brute force
  on tiny inputs) and never writes the padded tail;
* the printed communication figures (tests/golden/communication.tsv) and the
  peak-memory closed form.
"""
import math
import os

import numpy as np
import pytest

import oracle

U32 = 2.0 ** -24


def replicas_f16(psi, n, seed, std=1e-2):
    rng = np.random.default_rng(seed)
    return [(rng.standard_normal(psi) * std).astype(np.float16).view(np.uint16) for _ in range(n)]


@pytest.mark.parametrize("psi,n", [(1000, 8), (1003, 8), (10, 8), (4096, 1), (999, 64)])
@pytest.mark.parametrize("out_fmt", ["f32", "f16"])
def test_reduce_scatter_then_all_gather_is_all_reduce(psi, n, out_fmt):
    reps = replicas_f16(psi, n, psi + n)
    full = np.zeros(psi, np.float32)
    for r in reps:                         # all-reduce: sum of the full buffers, rank order
        full = full + oracle.decode16(r, "f16")
    shards = [oracle.reduce_shard(reps, "f16", out_fmt, psi, n, k) for k in range(n)]
    lay = oracle.layout(psi, n, 0)
    dt = np.float32 if out_fmt == "f32" else np.uint16
    out = np.full(lay.padded_total, 0x7E55 if dt == np.uint16 else np.nan, dt)
    oracle.gather_shards(shards, psi, n, out)
    want = full if out_fmt == "f32" else oracle.encode16(full, "f16")
    assert np.array_equal(out[:psi].view(np.uint8), want.view(np.uint8))
    # the padded tail is never written
    tail = out[psi:]
    assert (np.all(tail == 0x7E55) if dt == np.uint16 else np.all(np.isnan(tail)))


def test_reduce_identical_and_integer_replicas_exact():
    psi, n = 777, 8
    one = (np.random.default_rng(5).integers(-64, 65, psi) * 0.25).astype(np.float16)
    reps = [one.view(np.uint16).copy() for _ in range(n)]
    for r in range(n):
        got = oracle.reduce_shard(reps, "f16", "f32", psi, n, r)
        lay = oracle.layout(psi, n, r)
        assert np.array_equal(got, one[lay.offset:lay.offset + lay.count].astype(np.float32) * n)
    ints = [np.random.default_rng(k).integers(-100, 101, psi).astype(np.float16).view(np.uint16)
            for k in range(n)]
    exact = sum(x.view(np.float16).astype(np.int64) for x in ints)
    got = np.concatenate([oracle.reduce_shard(ints, "f16", "f32", psi, n, r) for r in range(n)])
    assert np.array_equal(got, exact[:got.size].astype(np.float32))


def test_reduce_within_summation_bound():
    psi, n = 3000, 16
    reps = replicas_f16(psi, n, 7, std=1.0)
    vals = np.stack([oracle.decode16(r, "f16").astype(np.float64) for r in reps])
    got = np.concatenate([oracle.reduce_shard(reps, "f16", "f32", psi, n, r) for r in range(n)])
    exact = np.array([math.fsum(c) for c in vals.T])
    bound = (n - 1) * U32 * np.abs(vals).sum(axis=0) * (1 + 1e-6)
    assert np.all(np.abs(got - exact) <= bound + 1e-45)


def test_reduce_bf16_in_f32_in():
    psi, n = 500, 4
    rng = np.random.default_rng(9)
    f = [rng.standard_normal(psi).astype(np.float32) for _ in range(n)]
    got = np.concatenate([oracle.reduce_shard(f, "f32", "f32", psi, n, r) for r in range(n)])
    assert np.array_equal(got, ((f[0] + f[1]) + f[2]) + f[3])
    b = [oracle.encode16(x, "bf16") for x in f]
    got = np.concatenate([oracle.reduce_shard(b, "bf16", "bf16", psi, n, r) for r in range(n)])
    ref = np.zeros(psi, np.float32)
    for x in b:
        ref = ref + oracle.decode16(x, "bf16")
    assert np.array_equal(got, oracle.encode16(ref, "bf16"))


def test_gather_brute_force_placement():
    for psi in range(1, 40):
        for n in range(1, 9):
            shards = [np.arange(1000 * k, 1000 * k + oracle.layout(psi, n, k).count,
                                dtype=np.float32) for k in range(n)]
            full = np.full(oracle.layout(psi, n, 0).padded_total, -1.0, np.float32)
            oracle.gather_shards(shards, psi, n, full)
            # element j of the flat buffer came from chunk j // S, position j % S
            S = oracle.layout(psi, n, 0).shard
            assert list(full[:psi]) == [1000 * (j // S) + (j % S) for j in range(psi)]
            assert np.all(full[psi:] == -1.0)


def _golden(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "communication.tsv")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            psi, d, q, printed, tol, src = line.rstrip("\n").split("\t")
            rows.append((int(psi), int(d), q, printed, float(tol), src))
    return rows


def test_printed_communication_figures(golden_dir):
    rows = _golden(golden_dir)
    assert len(rows) == 7
    for psi, d, q, printed, tol, src in rows:
        v0 = oracle.comm_volume(psi, d, 0, 2)
        if q == "ring_sent":
            value = v0["ring_bytes"] / 1e9
        elif q == "ring_bound":
            value = 2 * (2 * psi) / 1e9
            for dd in (2, 8, 64, 512, 4096):
                assert oracle.comm_volume(psi, dd, 0, 2)["ring_bytes"] < 2 * 2 * psi + 2 * 2 * dd
        elif q == "hops":
            value = v0["ring_hops"]
        elif q.startswith("wire_stage"):
            value = oracle.comm_volume(psi, d, int(q[-1]), 2)["wire_bytes"] / 1e9
        elif q == "ratio_3_vs_2":
            value = oracle.comm_volume(psi, d, 3, 2)["elements"] / v0["elements"]
        decimals = len(printed.split(".")[1]) if "." in printed else 0
        if tol == 0:
            assert round(value, decimals) == float(printed), (q, value, src)
        else:
            assert abs(value - float(printed)) <= tol, (q, value, src)


def test_stages_0_to_2_share_the_plain_volume():
    for psi, n in ((10**9, 8), (12345, 7)):
        vols = [oracle.comm_volume(psi, n, s, 2) for s in range(4)]
        assert vols[0] == vols[1] == vols[2]
        assert vols[3]["elements"] == 3 * psi and vols[0]["elements"] == 2 * psi
        assert vols[3]["ring_bytes"] * 2 == vols[0]["ring_bytes"] * 3


def test_peak_memory_closed_form():
    # 10B parameters over 64 GPUs: 2.5 GB persistent; one of 60 equal layers
    # gathered adds 1/60 of the 16-bit weights
    psi, n, layers = 10_000_000_000, 64, 60
    unit = psi // layers
    peak = oracle.peak_memory(psi, n, unit, 1, 0)
    assert peak == 16 * psi // n + 2 * unit
    assert round(oracle.layout(psi, n, 0).bytes_z3 / 1e9, 1) == 2.5
    # two units resident (one computed, one prefetched) and activations add linearly
    assert oracle.peak_memory(psi, n, unit, 2, 10**9) == 16 * psi // n + 4 * unit + 10**9
