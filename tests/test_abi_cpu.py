"""Host-side checks of the C ABI (no GPU needed).

* libzero_shard.so loads and exports every function include/zero_shard.h declares;
* the zero_layout struct has the same size and field offsets in C and in the binding;
* zero_shard_layout agrees with the oracle (and so with the brute force pinning it);
* argument errors come back as codes before anything touches a device;
* an empty rank's step returns OK without touching the device.
"""
import ctypes
import os
import re
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
import zero_sharded_mixed_shard_amd as zs
from zero_sharded_mixed_shard_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zero_shard.h")
TUNING_HEADER = os.path.join(ROOT, "include", "zero_shard_tuning.h")


def declared_functions(*headers):
    """Functions the given headers declare (default: every header under include/)."""
    if not headers:
        inc = os.path.join(ROOT, "include")
        headers = [os.path.join(inc, f) for f in sorted(os.listdir(inc)) if f.endswith(".h")]
    names = set()
    for h in headers:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"\b(zero_\w+)\s*\(", text))
    return sorted(names)


def test_product_header_holds_no_process_settings():
    # the launch-shape overrides live in the tuning header only
    product = declared_functions(HEADER)
    assert not [n for n in product if n.startswith("zero_set_")], product
    assert declared_functions(TUNING_HEADER) == ["zero_set_grid_cap", "zero_set_launch_piece",
                                                 "zero_set_occupancy"]


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("zero_shard_layout", "zero_overflow_check", "zero_adam_step",
                     "zero_strerror"):
        assert required in names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", zs.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(zs.lib, name)


def test_layout_struct_matches_header():
    src = r"""
    #include <stddef.h>
    #include <stdio.h>
    #include "zero_shard.h"
    int main(void) {
      printf("%zu", sizeof(zero_layout));
    #define F(f) printf(" %zu", offsetof(zero_layout, f));
      F(psi) F(shard) F(offset) F(count) F(pad) F(padded_total) F(n) F(rank)
      F(bytes_dp) F(bytes_z1) F(bytes_z2) F(bytes_z3)
      printf(" %d %d %d %d %d", ZERO_OK, ZERO_EINVAL, ZERO_EDTYPE, ZERO_EHIP, ZERO_SUMSQ_PARTIALS);
      return 0;
    }
    """
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        exe = os.path.join(d, "t")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-std=c11", "-I", os.path.dirname(HEADER), c, "-o", exe],
                       check=True)
        vals = [int(x) for x in subprocess.run([exe], capture_output=True, text=True,
                                               check=True).stdout.split()]
    size, offs, codes = vals[0], vals[1:13], vals[13:]
    S = _binding._Layout
    assert size == ctypes.sizeof(S)
    assert offs == [getattr(S, f).offset for f, _ in S._fields_]
    assert codes == [0, -1, -2, -3, _binding.SUMSQ_PARTIALS]


@pytest.mark.parametrize("psi,n", [(1, 1), (10, 8), (1_000_000, 8), (124_439_808, 8),
                                   (7_500_000_000, 8), (10_000_000_000, 1),
                                   (8_810_000_003, 64), (2**56, 3), (255, 32)])
def test_layout_matches_oracle(psi, n):
    for r in range(n):
        a = zs.zero_shard_layout(psi, n, r)
        b = oracle.layout(psi, n, r)
        assert a.__dict__ == b.__dict__


def test_layout_matches_oracle_small_exhaustive():
    for psi in range(1, 130):
        for n in range(1, 20):
            for r in range(n):
                assert zs.zero_shard_layout(psi, n, r).__dict__ == oracle.layout(psi, n, r).__dict__


@pytest.mark.parametrize("args", [(0, 8, 0), (10, 0, 0), (10, 8, 8), (2**56 + 1, 8, 0)])
def test_layout_errors(args):
    with pytest.raises(zs.ZeroError) as e:
        zs.zero_shard_layout(*args)
    assert e.value.code == -1
    assert zs.lib.zero_shard_layout(10, 8, 0, None) == -1


# Raw C calls with fake pointers: every one must be rejected (or be an empty
# rank) before any HIP call, so no device is needed.
FAKE = 0x10000  # never dereferenced
GOOD = dict(lr=1e-3, b1=0.9, b2=0.999, eps=1e-8, wd=0.0, step=1, S=1.0)


def adam(dt=0, psi=100, n=4, rank=0, ptrs=(FAKE,) * 5, flag=None, **kw):
    a = dict(GOOD, **kw)
    return zs.lib.zero_adam_step(*ptrs, dt, psi, n, rank, a["lr"], a["b1"], a["b2"], a["eps"],
                                 a["wd"], a["step"], a["S"], flag, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=2), -2), (dict(dt=-1), -2),
    (dict(psi=0), -1), (dict(n=0), -1), (dict(rank=4), -1), (dict(psi=2**56 + 1), -1),
    (dict(step=0), -1), (dict(S=0.0), -1), (dict(S=-1.0), -1), (dict(S=float("inf")), -1),
    (dict(S=float("nan")), -1), (dict(b1=1.0), -1), (dict(b1=-0.1), -1), (dict(b2=1.0), -1),
    (dict(b2=float("nan")), -1), (dict(eps=-1e-8), -1), (dict(eps=float("inf")), -1),
    (dict(lr=float("nan")), -1), (dict(wd=float("inf")), -1),
    (dict(ptrs=(None, FAKE, FAKE, FAKE, FAKE)), -1), (dict(ptrs=(FAKE, FAKE, None, FAKE, FAKE)), -1),
    (dict(ptrs=(FAKE, FAKE, FAKE, FAKE, None)), -1),
    (dict(ptrs=(FAKE + 1, FAKE, FAKE, FAKE, FAKE)), -1),      # w16 not 2-B aligned
    (dict(ptrs=(FAKE, FAKE, FAKE + 2, FAKE, FAKE)), -1),      # master not 4-B aligned
    (dict(flag=FAKE + 2), -1),
])
def test_adam_step_argument_errors(kw, code):
    assert adam(**kw) == code


def test_adam_step_empty_rank_is_a_no_op():
    # psi = 10 over 8 ranks: rank 7 owns nothing; null pointers are fine then
    assert adam(psi=10, n=8, rank=7, ptrs=(None,) * 5) == 0
    # but the scalars are still checked
    assert adam(psi=10, n=8, rank=7, ptrs=(None,) * 5, step=0) == -1


def check(dt=0, psi=100, n=4, rank=0, g=FAKE, S=1.0, flag=FAKE, sumsq=None, parts=None):
    return zs.lib.zero_overflow_check(g, dt, psi, n, rank, S, flag, sumsq, parts, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=5), -2), (dict(psi=0), -1), (dict(rank=9), -1), (dict(S=0.0), -1),
    (dict(S=float("inf")), -1), (dict(flag=None), -1), (dict(flag=FAKE + 1), -1),
    (dict(g=None), -1), (dict(g=FAKE + 1), -1), (dict(sumsq=FAKE), -1),
    (dict(sumsq=FAKE, parts=FAKE + 4), -1),
])
def test_overflow_check_argument_errors(kw, code):
    assert check(**kw) == code


def test_strerror():
    assert zs.zero_strerror(0) == "ok"
    assert "invalid" in zs.zero_strerror(-1)
    assert "dtype" in zs.zero_strerror(-2)
    assert "HIP" in zs.zero_strerror(-3)
    assert "unknown" in zs.zero_strerror(-99)


def test_binding_rejects_bad_tensors_before_the_library():
    import torch
    cpu = torch.zeros(10, dtype=torch.float16)
    with pytest.raises(ValueError):
        zs.zero_adam_step(cpu, cpu, torch.zeros(10), torch.zeros(10), torch.zeros(10), 10, 1, 0,
                          lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, step=1,
                          loss_scale=1.0)


def test_scaler_matches_oracle_policy_and_pages_trace():
    # the C5 schedule: overflow on every even step, S from 65536
    import numpy as np
    st = zs.Scaler(65536.0)
    ref = oracle.ScalerState(65536.0)
    applied = []
    for step in range(1, 11):
        found = int(step % 2 == 0)
        a = zs.zero_scaler_update(st, found)
        assert a == oracle.policy(ref, found)
        assert (st.step, st.loss_scale, st.clean_steps) == (ref.step, ref.loss_scale,
                                                             ref.clean_steps)
        if a:
            applied.append(st.step)
    assert applied == [1, 2, 3, 4, 5] and st.loss_scale == 2048.0
    # growth after a clean run, capped before it would overflow
    rng = np.random.default_rng(0)
    for interval in (0, 1, 3, 7):
        st = zs.Scaler(2.0 ** 120, growth_interval=interval)
        ref = oracle.ScalerState(2.0 ** 120, growth_interval=interval)
        for found in rng.integers(0, 2, 60) * (rng.random(60) < 0.3):
            assert zs.zero_scaler_update(st, int(found)) == oracle.policy(ref, int(found))
            assert (st.step, st.loss_scale, st.clean_steps) == (ref.step, ref.loss_scale,
                                                                 ref.clean_steps)
        assert np.isfinite(st.loss_scale)


def test_scaler_errors():
    st = zs.Scaler(0.0)
    with pytest.raises(zs.ZeroError):
        zs.zero_scaler_update(st, 0)
    st = zs.Scaler(float("inf"))
    with pytest.raises(zs.ZeroError):
        zs.zero_scaler_update(st, 1)
    assert zs.lib.zero_scaler_update(None, 0, None) == -1


def test_device_ctl_struct_matches_header():
    src = r"""
    #include <stddef.h>
    #include <stdio.h>
    #include "zero_shard.h"
    int main(void) {
      printf("%zu %zu", sizeof(zero_device_ctl), _Alignof(zero_device_ctl));
    #define F(f) printf(" %zu", offsetof(zero_device_ctl, f));
      F(scaler) F(found_inf) F(apply) F(loss_scale_used) F(bc1) F(bc2) F(status)
      F(rcp_loss_scale) F(rcp_bc1) F(rcp_bc2)
      printf(" %zu %d", sizeof(zero_scaler), ZERO_ERANGE);
      return 0;
    }
    """
    with tempfile.TemporaryDirectory() as d:
        c, exe = os.path.join(d, "t.c"), os.path.join(d, "t")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-std=c11", "-I", os.path.dirname(HEADER), c, "-o", exe],
                       check=True)
        vals = [int(x) for x in subprocess.run([exe], capture_output=True, text=True,
                                               check=True).stdout.split()]
    D = _binding.DeviceCtl
    assert vals[0] == ctypes.sizeof(D) and vals[1] == ctypes.alignment(D)
    assert vals[2:12] == [getattr(D, f).offset for f, _ in D._fields_]
    assert vals[12] == ctypes.sizeof(_binding.Scaler) and vals[13] == -4


@pytest.mark.parametrize("b1,b2,t0,n", [(0.9, 0.999, 1, 64), (0.9, 0.999, 101, 20),
                                        (0.95, 0.9999, 10_000, 7), (0.0, 0.5, 3, 5)])
def test_bias_table_matches_oracle_scalars(b1, b2, t0, n):
    tab = zs.zero_bias_corrections(b1, b2, t0, n).numpy()
    for k in range(n):
        ref = oracle.step_scalars(1e-3, b1, b2, 0.0, t0 + k)
        assert tab[k] == ref.bc1 and tab[n + k] == ref.bc2


def test_bias_table_errors():
    for args in ((0.9, 0.999, 0, 4), (1.0, 0.999, 1, 4), (0.9, -0.1, 1, 4)):
        with pytest.raises(zs.ZeroError):
            zs.zero_bias_corrections(*args)
    assert zs.lib.zero_bias_corrections(0.9, 0.999, 1, 0, FAKE) == -1
    assert zs.lib.zero_bias_corrections(0.9, 0.999, 1, 4, None) == -1


def test_device_path_argument_errors():
    L = zs.lib
    # check: dtype, layout, misaligned / null control block, null gradients
    assert L.zero_overflow_check_dev(FAKE, 3, 100, 4, 0, FAKE, None) == -2
    assert L.zero_overflow_check_dev(FAKE, 0, 100, 4, 4, FAKE, None) == -1
    assert L.zero_overflow_check_dev(FAKE, 0, 100, 4, 0, None, None) == -1
    assert L.zero_overflow_check_dev(FAKE, 0, 100, 4, 0, FAKE + 4, None) == -1
    assert L.zero_overflow_check_dev(None, 0, 100, 4, 0, FAKE, None) == -1
    # decision: null control block or table, empty table, t_first 0
    assert L.zero_scaler_update_dev(None, FAKE, 1, 4, None) == -1
    assert L.zero_scaler_update_dev(FAKE, None, 1, 4, None) == -1
    assert L.zero_scaler_update_dev(FAKE, FAKE, 1, 0, None) == -1
    assert L.zero_scaler_update_dev(FAKE, FAKE, 0, 4, None) == -1
    # step: as zero_adam_step, with the control block required
    p = (FAKE,) * 5
    assert L.zero_adam_step_dev(*p, 0, 100, 4, 0, 1e-3, 0.9, 0.999, 1e-8, 0.0, None, None) == -1
    assert L.zero_adam_step_dev(*p, 0, 100, 4, 0, 1e-3, 1.0, 0.999, 1e-8, 0.0, FAKE, None) == -1
    assert L.zero_adam_step_dev(*p, 2, 100, 4, 0, 1e-3, 0.9, 0.999, 1e-8, 0.0, FAKE, None) == -2
    # empty rank: no launch
    assert L.zero_adam_step_dev(None, None, None, None, None, 0, 10, 8, 7, 1e-3, 0.9, 0.999,
                                1e-8, 0.0, FAKE, None) == 0
    assert "table" in zs.zero_strerror(-4)


def test_fused_accumulate_check_argument_errors():
    L = zs.lib
    # dtype, layout, null or misaligned views and flag, bad S, overlaps -- all before any device call
    assert L.zero_grad_accumulate_check(FAKE * 4, FAKE, 3, 100, 4, 0, 1, 1.0, FAKE * 8, None) == -2
    assert L.zero_grad_accumulate_check(FAKE * 4, FAKE, 0, 100, 4, 4, 1, 1.0, FAKE * 8, None) == -1
    assert L.zero_grad_accumulate_check(None, FAKE, 0, 100, 4, 0, 1, 1.0, FAKE * 8, None) == -1
    assert L.zero_grad_accumulate_check(FAKE * 4, None, 0, 100, 4, 0, 1, 1.0, FAKE * 8, None) == -1
    assert L.zero_grad_accumulate_check(FAKE * 4 + 2, FAKE, 0, 100, 4, 0, 1, 1.0, FAKE * 8,
                                        None) == -1
    assert L.zero_grad_accumulate_check(FAKE * 4, FAKE, 0, 100, 4, 0, 1, 1.0, None, None) == -1
    assert L.zero_grad_accumulate_check(FAKE * 4, FAKE, 0, 100, 4, 0, 1, 1.0, FAKE * 8 + 2,
                                        None) == -1
    for S in (0.0, -1.0, float("inf"), float("nan")):
        assert L.zero_grad_accumulate_check(FAKE * 4, FAKE, 0, 100, 4, 0, 1, S, FAKE * 8,
                                            None) == -1
    # psi = 400 over 4 ranks: count 100; the flag inside acc, inside g16; acc over g16
    assert L.zero_grad_accumulate_check(FAKE * 4, FAKE, 0, 400, 4, 0, 0, 1.0, FAKE * 4 + 96,
                                        None) == -1
    assert L.zero_grad_accumulate_check(FAKE * 4, FAKE, 0, 400, 4, 0, 0, 1.0, FAKE + 100,
                                        None) == -1
    assert L.zero_grad_accumulate_check(FAKE + 100, FAKE, 0, 400, 4, 0, 0, 1.0, FAKE * 8,
                                        None) == -1
    # the device form: null or misaligned control block, or one inside a view
    assert L.zero_grad_accumulate_check_dev(FAKE * 4, FAKE, 0, 100, 4, 0, 1, None, None) == -1
    assert L.zero_grad_accumulate_check_dev(FAKE * 4, FAKE, 0, 100, 4, 0, 1, FAKE * 8 + 4,
                                            None) == -1
    assert L.zero_grad_accumulate_check_dev(FAKE * 4, FAKE, 0, 400, 4, 0, 1, FAKE * 4 + 64,
                                            None) == -1
    assert L.zero_grad_accumulate_check_dev(FAKE * 4, FAKE, 2, 100, 4, 0, 1, FAKE * 8,
                                            None) == -2


def test_fp32_gradient_device_path_argument_errors():
    L = zs.lib
    # check: layout, null or misaligned control block, null or misaligned gradients,
    # the control block inside the gradients
    assert L.zero_overflow_check_g32_dev(FAKE, 100, 4, 4, FAKE, None) == -1
    assert L.zero_overflow_check_g32_dev(FAKE, 100, 4, 0, None, None) == -1
    assert L.zero_overflow_check_g32_dev(FAKE, 100, 4, 0, FAKE + 4, None) == -1
    assert L.zero_overflow_check_g32_dev(None, 100, 4, 0, FAKE, None) == -1
    assert L.zero_overflow_check_g32_dev(FAKE + 2, 100, 4, 0, FAKE * 4, None) == -1
    assert L.zero_overflow_check_g32_dev(FAKE, 400, 4, 0, FAKE + 64, None) == -1
    # step: the control block is required, the hyperparameters and views are checked
    p = (FAKE, FAKE * 2, FAKE * 4, FAKE * 8, FAKE * 12)
    hp = (1e-3, 0.9, 0.999, 1e-8, 0.0)
    assert L.zero_adam_step_g32_dev(*p, 0, 100, 4, 0, *hp, None, None) == -1
    assert L.zero_adam_step_g32_dev(*p, 0, 100, 4, 0, 1e-3, 1.0, 0.999, 1e-8, 0.0, FAKE * 16,
                                    None) == -1
    assert L.zero_adam_step_g32_dev(*p, 2, 100, 4, 0, *hp, FAKE * 16, None) == -2
    assert L.zero_adam_step_g32_dev(FAKE, FAKE + 8, *p[2:], 0, 100, 4, 0, *hp, FAKE * 16,
                                    None) == -1                    # g32 overlaps w16
    assert L.zero_adam_step_g32_dev(*p, 0, 400, 4, 0, *hp, FAKE * 2 + 64, None) == -1
    # empty rank: no launch
    assert L.zero_adam_step_g32_dev(None, None, None, None, None, 0, 10, 8, 7, *hp, FAKE,
                                    None) == 0


@pytest.mark.parametrize("psi,n", [(8_810_000_000, 8), (8_810_000_000, 64), (10**9, 8),
                                   (12345, 7), (1, 1), (2**56, 4096)])
def test_comm_volume_matches_oracle(psi, n):
    for stage in range(4):
        for eb in (1, 2, 4, 8):
            assert zs.zero_comm_volume(psi, n, stage, eb) == oracle.comm_volume(psi, n, stage, eb)


def test_peak_memory_matches_oracle():
    for psi, n, unit, units, act in ((10**10, 64, 10**10 // 60, 1, 0), (10**10, 64, 10**8, 2, 5),
                                     (7_500_000_000, 8, 1, 0, 0), (12345, 7, 12345, 3, 99)):
        assert zs.zero_peak_memory(psi, n, unit, units, act) == \
            oracle.peak_memory(psi, n, unit, units, act)


def test_accounting_errors_and_struct():
    for args in ((0, 8, 0, 2), (10, 0, 0, 2), (10, 8, 4, 2), (10, 8, 0, 0), (10, 8, 0, 9)):
        with pytest.raises(zs.ZeroError):
            zs.zero_comm_volume(*args)
    with pytest.raises(zs.ZeroError):
        zs.zero_peak_memory(10, 2, 11, 1, 0)        # a unit larger than the model
    with pytest.raises(zs.ZeroError):
        zs.zero_peak_memory(2**56, 1, 2**56, 2**31, 2**63)   # overflow
    assert zs.lib.zero_comm_volume(10, 2, 0, 2, None) == -1
    src = r"""
    #include <stddef.h>
    #include <stdio.h>
    #include "zero_shard.h"
    int main(void) {
      printf("%zu %zu %zu %zu %zu %zu %d %d", sizeof(zero_comm), offsetof(zero_comm, collectives),
             offsetof(zero_comm, ring_hops), offsetof(zero_comm, elements),
             offsetof(zero_comm, wire_bytes), offsetof(zero_comm, ring_bytes),
             ZERO_MAX_LOCAL_RANKS, (int)ZERO_F32);
      return 0;
    }
    """
    with tempfile.TemporaryDirectory() as d:
        c, exe = os.path.join(d, "t.c"), os.path.join(d, "t")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-std=c11", "-I", os.path.dirname(HEADER), c, "-o", exe],
                       check=True)
        vals = [int(x) for x in subprocess.run([exe], capture_output=True, text=True,
                                               check=True).stdout.split()]
    C = _binding._Comm
    assert vals[0] == ctypes.sizeof(C)
    assert vals[1:6] == [getattr(C, f).offset for f, _ in C._fields_]
    assert vals[6] == _binding.MAX_LOCAL_RANKS and vals[7] == 2


def test_exchange_argument_errors():
    L = zs.lib
    arr = (ctypes.c_void_p * 4)(FAKE, FAKE, FAKE, FAKE)
    assert L.zero_reduce_shard(FAKE, 5, arr, 0, 100, 4, 0, None) == -2
    assert L.zero_reduce_shard(FAKE, 0, arr, 7, 100, 4, 0, None) == -2
    assert L.zero_reduce_shard(FAKE, 0, arr, 0, 100, 4, 4, None) == -1
    assert L.zero_reduce_shard(FAKE, 0, arr, 0, 100, 65, 0, None) == -1
    assert L.zero_reduce_shard(None, 0, arr, 0, 100, 4, 0, None) == -1
    assert L.zero_reduce_shard(FAKE + 2, 2, arr, 0, 100, 4, 0, None) == -1   # FP32 out misaligned
    bad = (ctypes.c_void_p * 4)(FAKE, None, FAKE, FAKE)
    assert L.zero_reduce_shard(FAKE, 0, bad, 0, 100, 4, 0, None) == -1
    assert L.zero_reduce_shard(None, 0, None, 0, 10, 8, 7, None) == 0        # empty rank
    assert L.zero_gather_shards(FAKE, arr, 3, 100, 4, None) == -2
    assert L.zero_gather_shards(None, arr, 0, 100, 4, None) == -1
    assert L.zero_gather_shards(FAKE, bad, 0, 100, 4, None) == -1
    assert L.zero_gather_shards(FAKE, arr, 0, 100, 65, None) == -1
    # the 16-bit-only entry points reject FP32
    assert L.zero_overflow_check(FAKE, 2, 100, 4, 0, 1.0, FAKE, None, None, None) == -2


def test_short_layout_name_is_the_same_call():
    for psi, n, rank in ((10, 8, 5), (1_000_003, 8, 7), (8_810_000_003, 64, 63)):
        assert zs.layout(psi, n, rank) == zs.zero_shard_layout(psi, n, rank)


def test_plain_c_client_links_and_calls_the_host_entry_points():
    # A C99 program with every warning an error, linked against the library,
    # drives the host-side entry points with no Python in between.
    src = r"""
    #include <inttypes.h>
    #include <stdio.h>
    #include <string.h>
    #include "zero_shard.h"
    int main(void) {
      zero_layout lay;
      if (zero_shard_layout(8810000003ULL, 64, 63, &lay) != ZERO_OK) return 1;
      printf("%" PRIu64 " %" PRIu64 " %" PRIu64 " %" PRIu64 "\n", lay.shard, lay.offset,
             lay.count, lay.pad);
      if (zero_shard_layout(10, 0, 0, &lay) != ZERO_EINVAL) return 2;
      zero_scaler sc;
      memset(&sc, 0, sizeof sc);
      sc.loss_scale = 65536.0f;
      sc.growth_interval = 2000;
      int32_t apply = -1;
      if (zero_scaler_update(&sc, 1, &apply) != ZERO_OK) return 3;
      printf("%d %g %" PRIu64 "\n", (int)apply, (double)sc.loss_scale, sc.step);
      if (zero_scaler_update(&sc, 0, &apply) != ZERO_OK) return 4;
      printf("%d %g %" PRIu64 "\n", (int)apply, (double)sc.loss_scale, sc.step);
      zero_comm c;
      if (zero_comm_volume(8810000003ULL, 64, 3, 2, &c) != ZERO_OK) return 5;
      printf("%u %" PRIu64 "\n", c.collectives, c.elements);
      float bc[4];
      if (zero_bias_corrections(0.9f, 0.999f, 1, 2, bc) != ZERO_OK) return 6;
      printf("%.9g %.9g %.9g %.9g\n", (double)bc[0], (double)bc[1], (double)bc[2],
             (double)bc[3]);
      printf("%s\n", zero_strerror(ZERO_EINVAL));
      return 0;
    }
    """
    lib_dir = os.path.dirname(zs.LIB_PATH)
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "client.c")
        exe = os.path.join(d, "client")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                        "-I", os.path.dirname(HEADER), c, "-o", exe, "-L", lib_dir,
                        "-lzero_shard", f"-Wl,-rpath,{lib_dir}"], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split("\n")
    lay = oracle.layout(8_810_000_003, 64, 63)
    assert out[0].split() == [str(lay.shard), str(lay.offset), str(lay.count), str(lay.pad)]
    assert out[1].split() == ["0", "32768", "0"]       # overflow: skip, S halves, t unchanged
    assert out[2].split() == ["1", "32768", "1"]       # clean: apply, t = 1
    assert out[3].split() == ["3", str(3 * 8_810_000_003)]
    b = [np.float32(x) for x in out[4].split()]        # %.9g round-trips FP32 exactly
    # 1 - beta^t with the FP32 beta widened to FP64, rounded once to FP32
    want = [np.float32(1.0 - float(np.float32(beta)) ** t) for beta in (0.9, 0.999) for t in (1, 2)]
    assert b == want
    assert out[5] == "invalid argument"


# Overlapping views are rejected before anything reaches a device.
@pytest.mark.parametrize("ptrs", [
    (FAKE, FAKE, FAKE * 4, FAKE * 8, FAKE * 12),             # w16 and g16 at one address
    (FAKE, FAKE * 2, FAKE * 4, FAKE * 4 + 396, FAKE * 12),   # m starts inside master's last element
    (FAKE * 16 + 8, FAKE * 2, FAKE * 4, FAKE * 8, FAKE * 16),  # w16 inside v
])
def test_adam_step_rejects_overlapping_views(ptrs):
    # psi = 400 over 4 ranks: count 100, so FP32 views span 400 bytes
    assert adam(psi=400, n=4, rank=0, ptrs=ptrs) == -1


def test_reduce_check_argument_errors():
    # psi = 400 over 4 ranks: rank 0's chunk is 100 elements (200 bytes of FP16)
    L = zs.lib
    reps = (ctypes.c_void_p * 4)(FAKE * 4, FAKE * 8, FAKE * 4, FAKE * 8)   # may repeat
    out, flag = FAKE * 12, FAKE * 16
    # the reduce's own errors come first
    assert L.zero_reduce_shard_check(out, 5, reps, 0, 400, 4, 0, 1.0, flag, None) == -2
    assert L.zero_reduce_shard_check(None, 0, reps, 0, 400, 4, 0, 1.0, flag, None) == -1
    assert L.zero_reduce_shard_check(out, 0, reps, 0, 400, 4, 4, 1.0, flag, None) == -1
    # the loss scale
    for S in (0.0, -1.0, float("inf"), float("nan")):
        assert L.zero_reduce_shard_check(out, 0, reps, 0, 400, 4, 0, S, flag, None) == -1
    # the flag: NULL, misaligned, inside the output, inside a replica's chunk
    assert L.zero_reduce_shard_check(out, 0, reps, 0, 400, 4, 0, 1.0, None, None) == -1
    assert L.zero_reduce_shard_check(out, 0, reps, 0, 400, 4, 0, 1.0, flag + 2, None) == -1
    assert L.zero_reduce_shard_check(out, 0, reps, 0, 400, 4, 0, 1.0, out + 196, None) == -1
    assert L.zero_reduce_shard_check(out, 0, reps, 0, 400, 4, 0, 1.0, FAKE * 8 + 100,
                                     None) == -1
    # the control block of the device-resident form: NULL, misaligned, over the output
    assert L.zero_reduce_shard_check_dev(out, 0, reps, 0, 400, 4, 0, None, None) == -1
    assert L.zero_reduce_shard_check_dev(out, 0, reps, 0, 400, 4, 0, flag + 4, None) == -1
    assert L.zero_reduce_shard_check_dev(out, 0, reps, 0, 400, 4, 0, out, None) == -1
    assert L.zero_reduce_shard_check_dev(out, 0, reps, 0, 400, 4, 0, FAKE * 4 + 64, None) == -1


def test_overlap_checks_of_accumulate_reduce_and_gather():
    # accumulate: acc (FP32) over the gradients
    assert zs.lib.zero_grad_accumulate(FAKE, FAKE + 200, 0, 400, 4, 0, 0, None) == -1
    # reduce: the output partly over one replica's chunk (rank 0: offset 0); exactly on
    # it (in place) is allowed
    reps = (ctypes.c_void_p * 2)(FAKE * 4, FAKE * 8)
    assert zs.lib.zero_reduce_shard(FAKE * 8 + 64, 0, reps, 0, 400, 4, 0, None) == -1
    # exactly on a replica's chunk but in a wider format: not in place, rejected
    assert zs.lib.zero_reduce_shard(FAKE * 8, 2, reps, 0, 400, 4, 0, None) == -1
    # gather: a shard overlapping the full buffer somewhere other than its own place
    shards = (ctypes.c_void_p * 4)(FAKE * 8, FAKE * 8 + 2, FAKE * 8 + 400, FAKE * 8 + 600)
    assert zs.lib.zero_gather_shards(FAKE * 8, shards, 0, 400, 4, None) == -1


def test_binding_rejects_host_tensors_before_any_device_call():
    # every device argument must be a device tensor: a host pointer reaching a
    # kernel would fault the GPU, so the binding refuses it first
    import torch
    n = 64
    h16 = torch.zeros(n, dtype=torch.float16)
    h32 = torch.zeros(n, dtype=torch.float32)
    flag = torch.zeros(1, dtype=torch.int32)
    ctl = torch.zeros(256, dtype=torch.uint8)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)
    calls = [
        lambda: zs.zero_overflow_check(h16, n, 1, 0, 1.0, flag),
        lambda: zs.zero_adam_step(h16, h16.clone(), h32, h32.clone(), h32.clone(), n, 1, 0,
                                  step=1, loss_scale=1.0, **hp),
        lambda: zs.zero_adam_step_g32(h16, h32, h32.clone(), h32.clone(), h32.clone(), n, 1, 0,
                                      step=1, loss_scale=1.0, **hp),
        lambda: zs.zero_grad_accumulate(h32, h16, n, 1, 0, first=True),
        lambda: zs.zero_overflow_check_g32(h32, n, 1, 0, 1.0, flag),
        lambda: zs.zero_overflow_check_dev(h16, n, 1, 0, ctl),
        lambda: zs.zero_scaler_update_dev(ctl, torch.zeros(8), 1),
        lambda: zs.zero_adam_step_dev(h16, h16.clone(), h32, h32.clone(), h32.clone(), n, 1, 0,
                                      ctl=ctl, **hp),
        lambda: zs.zero_reduce_shard(h16[:32], [h16, h16.clone()], n, 2, 0),
        lambda: zs.zero_reduce_shard_check(h16[:32], [h16, h16.clone()], n, 2, 0, 1.0, flag),
        lambda: zs.zero_reduce_shard_check_dev(h16[:32], [h16, h16.clone()], n, 2, 0, ctl),
        lambda: zs.zero_gather_shards(h16, [h16[:32].clone(), h16[:32].clone()], n, 2),
    ]
    for i, call in enumerate(calls):
        with pytest.raises(ValueError) as e:
            call()
        assert "device" in str(e.value), (i, str(e.value))


def test_library_depends_on_the_hip_runtime_only():
    # the boundary is plain C over HIP: no PyTorch library is linked into it
    out = subprocess.run(["readelf", "-d", zs.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    needed = re.findall(r"\(NEEDED\)\s+Shared library: \[([^\]]+)\]", out)
    assert any(n.startswith("libamdhip64") for n in needed), needed
    allowed = ("libamdhip64", "libstdc++", "libm.", "libgcc_s", "libc.", "ld-linux")
    assert all(n.startswith(allowed) for n in needed), needed
    assert not any("torch" in n or "c10" in n for n in needed), needed


def test_flag_control_and_check_outputs_may_not_overlap_the_views():
    # the step's skip flag inside master; the check's flag inside the gradients;
    # the partial sums over the flag
    assert adam(psi=400, n=4, rank=0, ptrs=(FAKE, FAKE * 2, FAKE * 4, FAKE * 8, FAKE * 12),
                flag=FAKE * 4 + 40) == -1
    assert check(psi=400, n=4, rank=0, g=FAKE * 4, flag=FAKE * 4 + 100) == -1
    assert check(psi=400, n=4, rank=0, g=FAKE * 4, flag=FAKE * 64, sumsq=FAKE * 96,
                 parts=FAKE * 64 - 8) == -1
    # the device control block inside the working weights
    assert zs.lib.zero_adam_step_dev(FAKE, FAKE * 2, FAKE * 4, FAKE * 8, FAKE * 12, 0, 400, 4, 0,
                                     1e-3, 0.9, 0.999, 1e-8, 0.0, FAKE + 64, None) == -1
    # the bias table over the control block the decision writes
    assert zs.lib.zero_scaler_update_dev(FAKE * 8, FAKE * 8 + 16, 1, 4, None) == -1


def test_tuning_setters_take_any_32_bit_value_and_the_binding_checks_range():
    # host-only stores; the kernels clamp what they read (grid cap: 1 .. 2^23
    # blocks, 0 = default; occupancy: 0 = by size, 8 and above = no cap)
    for v in (0, 1, 7, 8, 9, 2 ** 23, 2 ** 32 - 1):
        assert zs.lib.zero_set_grid_cap(v) == 0
        assert zs.lib.zero_set_occupancy(v) == 0
    for bad in (-1, 2 ** 32):
        with pytest.raises(ValueError):
            zs.zero_set_grid_cap(bad)
        with pytest.raises(ValueError):
            zs.zero_set_occupancy(bad)
    zs.zero_set_grid_cap(0)
    zs.zero_set_occupancy(0)
    # elements per launch: any 64-bit value (0 = each kernel's rule)
    for v in (0, 1, 2047, 2048, 1 << 28, 2 ** 64 - 1):
        assert zs.lib.zero_set_launch_piece(v) == 0
    for bad in (-1, 2 ** 64):
        with pytest.raises(ValueError):
            zs.zero_set_launch_piece(bad)
    zs.zero_set_launch_piece(0)
