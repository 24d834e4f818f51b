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


def write_profile(path, symbol, isa, workload, traffic):
    with open(path, "w") as f:
        f.write("# test profile\n\n")
        f.write(f"- kernel_symbol: `{symbol}`\n- kernel_isa_sha256: `{isa}`\n")
        f.write(f"- workload: {workload}\n- hbm_bytes_per_launch: {traffic:.6e}\n")


def test_traffic_used_only_for_matching_code_and_workload(bench, hashes, tmp_path, monkeypatch):
    sym = step_symbol(hashes, 0)
    prof = tmp_path / "p.md"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(prof))
    write_profile(prof, sym, hashes[sym], "flat10B_n1_f16_adamw", 2.8e11)
    assert bench.measured_traffic("flat10B_n1_f16_adamw") == pytest.approx(2.8e11)
    assert bench.measured_traffic("other_workload") is None
    write_profile(prof, sym, "0" * 64, "flat10B_n1_f16_adamw", 2.8e11)
    assert bench.measured_traffic("flat10B_n1_f16_adamw") is None
    write_profile(prof, step_symbol(hashes, 1), hashes[sym], "flat10B_n1_f16_adamw", 2.8e11)
    assert bench.measured_traffic("flat10B_n1_f16_adamw") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.md"))
    assert bench.measured_traffic("flat10B_n1_f16_adamw") is None
