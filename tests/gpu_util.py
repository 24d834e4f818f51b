"""Helpers of the GPU parity tests: shard buffers with guard elements, the
parity bar, and host copies of windows.

The parity bar: master, m and v within 2 ulp of the oracle (ordinal distance
of the bit patterns, +0 == -0), the 16-bit working weights within 1 ulp, and
the overflow flag and layouts bit-exact.  Guard elements around every view
must come back untouched.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import synth

TOL_F32_ULP = 2
TOL_16_ULP = 1
GUARD = 24                       # guard elements on each side of a view
SENT16 = 0x7E55                  # NaN-pattern sentinel in 16-bit guards
SENT32 = np.uint32(0x7FC0DEAD)   # NaN-pattern sentinel in FP32 guards

HP_KEYS = ("lr", "beta1", "beta2", "eps", "weight_decay")


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def u16(t: torch.Tensor) -> np.ndarray:
    return synth.to_numpy_u16(t)


def f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.float32, copy=True)


class GuardedView:
    """A 1-D device view of `count` elements at element `phase` of a 16-B-aligned
    allocation, with GUARD sentinel elements before and after it."""

    def __init__(self, count: int, dtype: torch.dtype, phase: int, device):
        self.count, self.phase = count, phase
        self.buf = torch.empty(phase + GUARD + count + GUARD, dtype=dtype, device=device)
        assert self.buf.data_ptr() % 256 == 0
        if dtype == torch.float32:
            self.buf.view(torch.int32).fill_(int(SENT32.view(np.int32)))
        else:
            self.buf.view(torch.int16).fill_(int(np.uint16(SENT16).view(np.int16)))
        self.start = phase + GUARD
        self.view = self.buf[self.start:self.start + count]

    def guards_intact(self) -> bool:
        raw = self.buf.view(torch.int32 if self.buf.dtype == torch.float32 else torch.int16)
        raw = raw.cpu().numpy()
        want = SENT32.view(np.int32) if self.buf.dtype == torch.float32 else \
            np.uint16(SENT16).view(np.int16)
        before = raw[self.start - GUARD:self.start]
        after = raw[self.start + self.count:]
        return bool(np.all(before == want) and np.all(after == want))


def line_head(phase: int, elem_bytes: int, line: int = 128) -> int:
    """Elements a kernel does one at a time before the first cache-line boundary
    of a GuardedView at `phase` (its view starts phase + GUARD elements into a
    256-B aligned allocation)."""
    start = (phase + GUARD) * elem_bytes
    return ((line - start % line) % line) // elem_bytes


def _distance_where_bits_differ(a: np.ndarray, b: np.ndarray, bits, ulp) -> tuple:
    """(max ulp distance, elements at a nonzero distance): the ulp distance is taken only
    where the bit patterns differ (equal patterns are at distance 0), which keeps
    comparisons of whole full-size shards cheap."""
    a = np.ascontiguousarray(a).view(bits)
    b = np.ascontiguousarray(b).view(bits)
    assert a.shape == b.shape, (a.shape, b.shape)
    idx = np.flatnonzero(a != b)
    if idx.size == 0:
        return 0, 0
    d = ulp(a[idx], b[idx])
    return int(d.max()), int(np.count_nonzero(d))


def assert_close(gpu: dict, ref: dict, dtype: str, what: str = "") -> dict:
    """Apply the parity bar to host copies {master, m, v, w16}; return statistics."""
    stats = {}
    for k in ("master", "m", "v"):
        stats[k] = _distance_where_bits_differ(
            gpu[k], ref[k], np.uint32,
            lambda x, y: oracle.ulp_distance32(x.view(np.float32), y.view(np.float32)))
        assert stats[k][0] <= TOL_F32_ULP, (what, k, stats[k])
    stats["w16"] = _distance_where_bits_differ(
        gpu["w16"], ref["w16"], np.uint16, lambda x, y: oracle.ulp_distance16(x, y, dtype))
    assert stats["w16"][0] <= TOL_16_ULP, (what, "w16", stats["w16"])
    return stats


def hp_of(w) -> dict:
    return {k: getattr(w, k) for k in HP_KEYS}
