"""The allocation-free overflow check against the one that takes a workspace.

zero_overflow_check_noalloc keeps the sum of squares' partial sums in the
library's fixed per-device array instead of a caller buffer.  Called through
the C ABI, its flag and sum of squares must equal zero_overflow_check's bit
for bit on the same gradients -- on two calls in a row, the second with a
smaller input (the array keeps the first call's contents), in both 16-bit
formats, with the flag raised and not, and without a sum of squares.
"""
import ctypes

import numpy as np
import pytest
import torch

import synth
import zero_sharded_mixed_shard_amd as zs
from gpu_util import GuardedView, log

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TD = {"f16": torch.float16, "bf16": torch.bfloat16}
FMT = {"f16": 0, "bf16": 1}


def both(g: GuardedView, count: int, dtype: str, S: float, with_sumsq: bool):
    """(flag, sumsq bits) from the workspace form and from the allocation-free form."""
    out = []
    for form in ("workspace", "noalloc"):
        flag = torch.full((1,), 7, dtype=torch.int32, device=DEV)
        sumsq = torch.full((1,), -1.0, dtype=torch.float32, device=DEV) if with_sumsq else None
        p_s = sumsq.data_ptr() if with_sumsq else None
        if form == "workspace":
            parts = torch.empty(zs.SUMSQ_PARTIALS, dtype=torch.float64, device=DEV)
            rc = zs.lib.zero_overflow_check(g.view.data_ptr(), FMT[dtype], count, 1, 0, S,
                                            flag.data_ptr(), p_s,
                                            parts.data_ptr() if with_sumsq else None, None)
        else:
            rc = zs.lib.zero_overflow_check_noalloc(g.view.data_ptr(), FMT[dtype], count, 1, 0,
                                                    S, flag.data_ptr(), p_s, None)
        assert rc == 0, (form, zs.zero_strerror(rc))
        torch.cuda.synchronize()
        bits = int(sumsq.view(torch.int32).item()) if with_sumsq else None
        out.append((int(flag.item()), bits))
    return out


def make_grads(count, dtype, phase, seed, inject):
    g = synth.fill_normal_(torch.empty(count, dtype=TD[dtype]), 1e-2, seed)
    if inject:
        g[count // 3] = float("nan")
    view = GuardedView(count, TD[dtype], phase, DEV)
    view.view.copy_(g.to(DEV))
    return view


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_noalloc_check_equals_the_workspace_form_on_two_calls(dtype):
    # a large call, then a smaller one at another phase and scale; then a
    # flag-raising call and a flag-only call
    cases = [(3_000_017, 1, 3.0, False, True), (1_000, 5, 1024.0, False, True),
             (70_001, 2, 65536.0, True, True), (4_097, 0, 1.0, False, False)]
    for i, (count, phase, S, inject, with_sumsq) in enumerate(cases):
        g = make_grads(count, dtype, phase, 31_000 + i, inject)
        ws, na = both(g, count, dtype, S, with_sumsq)
        log(f"noalloc {dtype} count={count} S={S} sumsq={with_sumsq}: {ws} / {na}")
        assert ws == na, (dtype, count, S, ws, na)
        assert ws[0] == int(inject)
        if with_sumsq and not inject:
            assert ws[1] != int(np.float32(-1.0).view(np.int32))   # the sum was written
        assert g.guards_intact()


def test_noalloc_check_argument_errors_come_back_before_any_launch():
    g = torch.zeros(16, dtype=torch.float16, device=DEV)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    lib = zs.lib
    assert lib.zero_overflow_check_noalloc(g.data_ptr(), 0, 16, 1, 0, 0.0, flag.data_ptr(),
                                           None, None) == -1          # S = 0
    assert lib.zero_overflow_check_noalloc(g.data_ptr(), 5, 16, 1, 0, 1.0, flag.data_ptr(),
                                           None, None) == -2          # bad format
    assert lib.zero_overflow_check_noalloc(g.data_ptr(), 0, 16, 1, 0, 1.0, None, None,
                                           None) == -1                # no flag
    assert lib.zero_overflow_check_noalloc(g.data_ptr(), 0, 16, 1, 0, 1.0, g.data_ptr(),
                                           None, None) == -1          # flag inside g
    torch.cuda.synchronize()
