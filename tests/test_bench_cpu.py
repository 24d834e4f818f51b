"""Host-side checks of bench.py's bookkeeping (no GPU needed).

* the build records a machine-code hash for every kernel, the step kernels included;
* the counter-measured traffic is used only when the profile names this workload and
  the same machine code of the step kernel as the library built now.
"""
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load(path, name):
    spec = importlib.util.spec_from_file_location(name, path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="module")
def bench():
    return load(os.path.join(ROOT, "bench.py"), "bench_under_test")


@pytest.fixture(scope="module")
def hashes():
    b = load(os.path.join(ROOT, "zero_sharded_mixed_shard_amd", "build.py"), "zs_build_t")
    h = b.read_isa_hashes()
    if not h:
        pytest.skip("library not built (no kernel hashes beside it)")
    return h


def step_symbol(hashes, dt):
    # the vector step with 16-bit gradients and S a power of two (the benchmarked one)
    names = [k for k in hashes if f"adam_step_vecILi{dt}EtLi2ELi0EE" in k]
    assert len(names) == 1, names
    return names[0]


def test_every_step_kernel_has_a_hash(hashes):
    for dt in (0, 1):
        assert len(hashes[step_symbol(hashes, dt)]) == 64
    for part in ("overflow_flag_kernel", "accumulate_vec", "reduce_shard_kernel", "gather_kernel",
                 "scaler_decide"):
        assert any(part in k for k in hashes), part
    # the two formats compile to different code
    assert hashes[step_symbol(hashes, 0)] != hashes[step_symbol(hashes, 1)]


def write_profile(path, symbol, isa, workload, traffic, launches=75):
    with open(path, "w") as f:
        f.write("# test profile\n\n")
        f.write(f"- kernel_symbol: `{symbol}`\n- kernel_isa_sha256: `{isa}`\n")
        f.write(f"- workload: {workload}\n- launches_per_step: {launches}\n")
        f.write(f"- hbm_bytes_per_step: {traffic:.6e}\n")


def test_traffic_used_only_for_matching_code_and_workload(bench, hashes, tmp_path, monkeypatch):
    sym = step_symbol(hashes, 0)
    prof = tmp_path / "p.md"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(prof))
    write_profile(prof, sym, hashes[sym], "flat10B_n1_f16_adamw", 2.8e11)
    assert bench.measured_traffic("flat10B_n1_f16_adamw") == pytest.approx(2.8e11)
    assert bench.launches_per_step("flat10B_n1_f16_adamw") == 75
    assert bench.measured_traffic("other_workload") is None
    assert bench.launches_per_step("other_workload") is None
    write_profile(prof, sym, "0" * 64, "flat10B_n1_f16_adamw", 2.8e11)
    assert bench.measured_traffic("flat10B_n1_f16_adamw") is None
    write_profile(prof, step_symbol(hashes, 1), hashes[sym], "flat10B_n1_f16_adamw", 2.8e11)
    assert bench.measured_traffic("flat10B_n1_f16_adamw") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.md"))
    assert bench.measured_traffic("flat10B_n1_f16_adamw") is None


def test_parity_windows_cover_head_tail_and_past_2e32(bench):
    wins = bench.parity_windows(10_000_000_000, seed=4)
    w = bench.PARITY_WINDOW
    assert wins[0] == (0, w) and wins[-1] == (10_000_000_000 - w, 10_000_000_000)
    assert (1 << 32, (1 << 32) + w) in wins
    assert len(wins) == 3 + bench.PARITY_RANDOM
    assert all(b - a == w and 0 <= a < b <= 10_000_000_000 for a, b in wins)
    assert wins == sorted(wins)
    # a shard smaller than a window: one window, the whole shard
    assert bench.parity_windows(1000, seed=1) == [(0, 1000)]


def test_replay_parity_reports_zero_ulp_on_oracle_data_and_finds_a_flipped_bit(bench):
    import numpy as np

    import oracle
    import synth

    w = synth.WORKLOADS[4]
    rng = np.random.default_rng(3)
    start, final = [], []
    applied = [(1, 65536.0), (2, 65536.0), (3, 32768.0)]
    for _ in range(3):
        n = 1000
        s0 = {"g16": (rng.standard_normal(n) * 1e-3 * 65536).astype(np.float16).view(np.uint16),
              "master": (rng.standard_normal(n) * 0.02).astype(np.float32),
              "m": np.zeros(n, np.float32), "v": np.zeros(n, np.float32),
              "w16": np.zeros(n, np.uint16)}
        s1 = {k: s0[k].copy() for k in s0}
        hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay)
        for t, S in applied:
            oracle.adam_step(s1["w16"], s0["g16"], s1["master"], s1["m"], s1["v"], "f16",
                             step=t, loss_scale=S, **hp)
        start.append(s0)
        final.append(s1)
    r = bench.replay_parity(w, start, final, applied, [(0, 0)] * 4)
    assert r["ok"] and r["max_ulp"] == {"master": 0, "m": 0, "v": 0, "w16": 0}
    assert r["non_bitwise"] == {"master": 0, "m": 0, "v": 0, "w16": 0}
    assert r["elements"] == 3000 and r["steps_replayed"] == 3
    final[1]["m"][17] = np.nextafter(final[1]["m"][17], np.float32(1))
    final[2]["master"][5] = np.float32(final[2]["master"][5] * 1.01)
    r = bench.replay_parity(w, start, final, applied, [(0, 0), (1, 0)])
    assert not r["ok"] and not r["flags_equal"]
    assert r["max_ulp"]["m"] == 1 and r["non_bitwise"]["m"] == 1
    assert r["max_ulp"]["master"] > 2 and r["non_bitwise"]["master"] == 1


def test_bench_layout_parity_covers_every_rank(bench):
    for psi, n in ((10_000_000_000, 1), (7_500_000_000, 8), (8_810_000_003, 64), (1_500_000_000, 1)):
        assert bench.layouts_equal(psi, n)
