"""Checks on the gfx950 assembly of our own kernels (host only: hipcc cross-compiles).

The numerics contract needs correctly rounded FP32 division and square root,
round-to-nearest-even 16-bit conversions and no packed FP32 VALU ops; the
memory contract needs 16-byte vector loads and stores in the step, and no
scalar-cache writes anywhere.
"""
import re

import pytest

ROOT_BUILD = None


@pytest.fixture(scope="module")
def asm():
    import importlib.util
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    spec = importlib.util.spec_from_file_location(
        "_zs_build", os.path.join(root, "zero_sharded_mixed_shard_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    text = mod.device_assembly()
    kernels = {}
    for m in re.finditer(r"^(_Z\S+):[^\n]*\n(.*?)^\.Lfunc_end", text, re.M | re.S):
        kernels[m.group(1)] = m.group(2)
    assert kernels
    return text, kernels


def count(body, op):
    return len(re.findall(r"\b" + re.escape(op) + r"\b", body))


def test_no_forbidden_instructions(asm):
    text, _ = asm
    for op in ("v_pk_fma_f32", "v_pk_mul_f32", "v_pk_add_f32", "v_cvt_pkrtz_f16_f32",
               "s_store_dword", "s_store_dwordx2", "s_store_dwordx4", "s_atomic_add",
               "s_dcache_wb", "s_dcache_discard", "s_buffer_store_dword"):
        assert count(text, op) == 0, op
    assert not re.search(r"\bs_(store|atomic|buffer_store|buffer_atomic|scratch_store)\w*", text)
    assert not re.search(r"\bs_dcache_(wb|discard)\w*", text)


# per element of the step, by unscale mode (0: S a power of two, multiply by
# the exact 1/S; 1: FP64 reciprocal product; 2: the device control block picks
# one of the two bodies): FP32 divisions (the update's (lr*m^)/den, and one
# guarded fallback per quotient formed as an FP64 product) and FP64 products
DIVS_PER_ELEM = {0: 3, 1: 4}
PRODUCTS_PER_ELEM = {0: 2, 1: 3}
STEP_NAME = re.compile(r"adam_step_(vec|elem)ILi(\d)E([tf])(?:Li2E)?Li(\d)EE")


def test_step_kernels_keep_each_operation_correctly_rounded(asm):
    _, kernels = asm
    steps = {k: b for k, b in kernels.items() if "adam_step" in k}
    # vector and element-wise kernels x FP16 / BF16 weights x 16-bit / FP32
    # gradients x three unscale modes
    assert len(steps) == 24
    for name, body in steps.items():
        mode = int(STEP_NAME.search(name).group(4))
        modes = (0, 1) if mode == 2 else (mode,)
        sq = count(body, "v_sqrt_f32_e32") + count(body, "v_sqrt_f32_e64")
        assert sq >= len(modes) and sq % len(modes) == 0, name
        per_body = sq // len(modes)         # element bodies: tile elements, head, tail
        # every division left is the full scale / reciprocal / fma / fixup sequence
        divs = sum(DIVS_PER_ELEM[md] for md in modes) * per_body
        assert count(body, "v_div_fixup_f32") == divs, name
        assert count(body, "v_div_fmas_f32") == divs, name
        # each constant-divisor quotient: widen, one FP64 product, one rounding
        prods = sum(PRODUCTS_PER_ELEM[md] for md in modes) * per_body
        assert count(body, "v_mul_f64") == prods, name
        assert count(body, "v_cvt_f32_f64_e32") == prods, name
        assert count(body, "v_div_fixup_f64") == 0, name   # reciprocals come from the host
        # the square root is refined to the correctly rounded result
        assert count(body, "v_cmp_class_f32_e32") + count(body, "v_cmp_class_f32_e64") >= sq
        if "ILi0E" in name:      # FP16 (the SDWA form writes the upper half-word)
            assert sum(count(body, "v_cvt_f16_f32_" + f) for f in ("e32", "e64", "sdwa")) == sq
        else:                    # BF16: gfx950's round-to-nearest-even convert
            assert count(body, "v_cvt_pk_bf16_f32") == sq


def test_vector_step_uses_16_byte_accesses(asm):
    _, kernels = asm
    vec = {k: b for k, b in kernels.items() if "adam_step_vec" in k}
    assert len(vec) == 12
    for name, body in vec.items():
        g32 = "EfLi" in name     # FP32 gradients: one more 16-B load per group
        assert count(body, "global_load_dwordx4") >= (8 if g32 else 6)  # master, m, v (, g)
        assert count(body, "global_store_dwordx4") >= 6
        if not g32:
            assert count(body, "global_load_dwordx2") >= 2  # 4 gradients per lane per group
        assert count(body, "global_store_dwordx2") >= 2     # 4 working weights
    acc = {k: b for k, b in kernels.items() if "accumulate_vec" in k}
    assert len(acc) == 8       # FP16 / BF16 x first / not x with / without the fused check
    for name, body in acc.items():
        assert count(body, "global_store_dwordx4") >= 2
        if "Lb0ELi2ELb0E" in name or "Lb0ELi2ELb1E" in name:   # not the first micro-batch
            assert count(body, "global_load_dwordx4") >= 2


def test_sum_of_squares_visits_every_vector_lane(asm):
    # each lane's 16-B vectors hold 8 (16-bit) or 4 (FP32) gradients; each is
    # visited once in each of two paths (4 vectors in flight + 1 remainder
    # vector + the scalar head and tail = n visits per path).  S a power of
    # two: multiply by 1/S in FP32, widen, one FP64 FMA.  Any other S: widen,
    # one FP64 multiply by RN64(1/S), one rounding to FP32, widen again, one
    # FP64 FMA -- and, in the branch a vector takes when a quotient is below
    # 2^-125 (zeros included), one guarded FP32 divide per gradient.  Plus the
    # two reciprocals (FP32 and FP64) once per lane.
    _, kernels = asm
    sumsq = {k: b for k, b in kernels.items() if "overflow_sumsq_kernel" in k}
    assert len(sumsq) == 3
    for name, body in sumsq.items():
        per_vec = 4 if "IfLi" in name else 8
        n = 5 * per_vec + 2
        assert count(body, "v_cvt_f64_f32_e32") == 3 * n + 1, name
        assert count(body, "v_cvt_f32_f64_e32") == n, name
        assert count(body, "v_mul_f64") == n + 1, name          # + one inside 1/S in FP64
        assert count(body, "v_fmac_f64_e32") == 2 * n, name     # the squares, both paths
        assert count(body, "v_div_fixup_f64") == 1, name        # RN64(1/S), once
        assert count(body, "v_div_fixup_f32") == n + 1, name    # the fallback divides, and 1/S
        assert count(body, "global_load_dwordx4") == 10, name
        assert count(body, "v_mov_b32_dpp") == 12, name        # wave sum: 6 DPP steps x 2 halves
