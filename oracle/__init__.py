"""Plain CPU oracle for the ZeRO-sharded mixed-precision Adam step.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import this package.  It
shares no code with the HIP library and imports nothing from it; the two meet
only in the seeded input generators of ``synth``.

The arithmetic lives in ``oracle.c`` (scalar C, one IEEE binary32 operation
at a time) and is reached through ctypes; this module adds argument
marshalling and the host-side loss-scale policy.

Sources (page title, section):
  * "Training models too big for one GPU: ZeRO & FSDP" -- "Adam, and why it's
    expensive" (update equations), "How a computer stores real numbers"
    (format table), "Mixed-precision training" (FP32 master copy, loss
    scaling, skip on overflow), "The memory bill: 16 bytes per parameter",
    "Data parallelism and the all-reduce" (chunk i to GPU i), "ZeRO stages 1,
    2 and 3" (per-GPU formulas).
  * "Stop Replicating What You Can Shard: ZeRO and FSDP" -- "The three stages
    of ZeRO".
  * "ZeRO memory math" (tm_zero_math) -- "Stage 1 - P_os" (N equal shards).
  * "ZeRO Stage 3 Math" -- "Stage 3: divide everything by N".

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
except the FP64 sum of squares (``overflow_check(...)[1]``), whose only pin is
an exactly rounded sum (``math.fsum``) of the same squares; the pages never
define a gradient norm.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DTYPES = {"f16": 0, "bf16": 1}



def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no HIP, no FMA); see build_oracle.py."""
    if force or not os.path.exists(_LIB):
        from . import build_oracle
        build_oracle.build()
    return _LIB


class _Layout(ctypes.Structure):
    _fields_ = [
        ("psi", ctypes.c_uint64),
        ("shard", ctypes.c_uint64),
        ("offset", ctypes.c_uint64),
        ("count", ctypes.c_uint64),
        ("pad", ctypes.c_uint64),
        ("padded_total", ctypes.c_uint64),
        ("n", ctypes.c_uint32),
        ("rank", ctypes.c_uint32),
        ("bytes_dp", ctypes.c_uint64),
        ("bytes_z1", ctypes.c_uint64),
        ("bytes_z2", ctypes.c_uint64),
        ("bytes_z3", ctypes.c_uint64),
    ]


class _Scalars(ctypes.Structure):
    _fields_ = [(k, ctypes.c_float) for k in ("bc1", "bc2", "omb1", "omb2", "decay")]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        u64, u32, i32, f32, f64 = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int,
                                   ctypes.c_float, ctypes.c_double)
        vp = ctypes.c_void_p
        lib.oracle_layout.argtypes = [u64, u32, u32, ctypes.POINTER(_Layout)]
        lib.oracle_layout.restype = i32
        lib.oracle_decode16.argtypes = [ctypes.c_uint16, i32]
        lib.oracle_decode16.restype = f64
        lib.oracle_encode16.argtypes = [f64, i32]
        lib.oracle_encode16.restype = ctypes.c_uint16
        lib.oracle_decode16_array.argtypes = [vp, vp, u64, i32]
        lib.oracle_encode16_array.argtypes = [vp, vp, u64, i32]
        lib.oracle_overflow_check.argtypes = [vp, i32, u64, f32, vp, vp]
        lib.oracle_step_scalars.argtypes = [f32, f32, f32, f32, u64, ctypes.POINTER(_Scalars)]
        lib.oracle_adam_step.argtypes = [vp, vp, vp, vp, vp, i32, u64, f32, f32, f32, f32, f32,
                                         u64, f32]
        lib.oracle_adam_step_f64.argtypes = [vp, vp, vp, vp, i32, u64, f64, f64, f64, f64, f64,
                                             u64, f64]
        lib.oracle_grad_accumulate.argtypes = [vp, vp, i32, u64, i32]
        lib.oracle_overflow_check_g32.argtypes = [vp, u64, f32, vp, vp]
        lib.oracle_adam_step_g32.argtypes = [vp, vp, vp, vp, vp, i32, u64, f32, f32, f32, f32,
                                             f32, u64, f32]
        lib.oracle_reduce_shard.argtypes = [vp, i32, vp, i32, u64, u32, u32]
        lib.oracle_gather_shards.argtypes = [vp, vp, i32, u64, u32]
        lib.oracle_reduce_shard.restype = None
        lib.oracle_gather_shards.restype = None
        for name in ("oracle_decode16_array", "oracle_encode16_array", "oracle_overflow_check",
                     "oracle_step_scalars", "oracle_adam_step", "oracle_adam_step_f64",
                     "oracle_grad_accumulate", "oracle_overflow_check_g32",
                     "oracle_adam_step_g32"):
            getattr(lib, name).restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray, dtype) -> int:
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    if not a.flags.c_contiguous:
        raise ValueError("oracle arrays must be C-contiguous")
    return a.ctypes.data


@dataclass(frozen=True)
class Layout:
    psi: int
    shard: int
    offset: int
    count: int
    pad: int
    padded_total: int
    n: int
    rank: int
    bytes_dp: int
    bytes_z1: int
    bytes_z2: int
    bytes_z3: int


def layout(psi: int, n: int, rank: int) -> Layout:
    """Shard layout of rank ``rank`` among ``n`` over a flat buffer of ``psi`` params."""
    out = _Layout()
    rc = _load().oracle_layout(psi, n, rank, ctypes.byref(out))
    if rc != 0:
        raise ValueError(f"invalid layout arguments psi={psi} n={n} rank={rank}")
    return Layout(*(getattr(out, f) for f, _ in _Layout._fields_))


def decode16(bits: np.ndarray, dtype: str) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, np.float32)
    _load().oracle_decode16_array(_ptr(bits, np.uint16), _ptr(out, np.float32), bits.size,
                                  DTYPES[dtype])
    return out


def encode16(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().oracle_encode16_array(_ptr(x, np.float32), _ptr(out, np.uint16), x.size,
                                  DTYPES[dtype])
    return out


def overflow_check(g16: np.ndarray, dtype: str, loss_scale: float) -> tuple[int, float]:
    """Return (found_inf, sum of squares of the unscaled gradients)."""
    flag = np.zeros(1, np.int32)
    s = np.zeros(1, np.float64)
    _load().oracle_overflow_check(_ptr(g16, np.uint16), DTYPES[dtype], g16.size, loss_scale,
                                  flag.ctypes.data, s.ctypes.data)
    return int(flag[0]), float(s[0])


@dataclass(frozen=True)
class Scalars:
    bc1: float
    bc2: float
    omb1: float
    omb2: float
    decay: float


def step_scalars(lr, beta1, beta2, weight_decay, step) -> Scalars:
    out = _Scalars()
    _load().oracle_step_scalars(lr, beta1, beta2, weight_decay, step, ctypes.byref(out))
    return Scalars(out.bc1, out.bc2, out.omb1, out.omb2, out.decay)


def adam_step(w16, g16, master, m, v, dtype, *, lr, beta1, beta2, eps, weight_decay, step,
              loss_scale) -> None:
    """One Adam step over a shard, in place on numpy arrays of equal length."""
    count = g16.size
    for a in (w16, master, m, v):
        if a.size != count:
            raise ValueError("all shard arrays must have the same length")
    _load().oracle_adam_step(_ptr(w16, np.uint16), _ptr(g16, np.uint16), _ptr(master, np.float32),
                             _ptr(m, np.float32), _ptr(v, np.float32), DTYPES[dtype], count,
                             lr, beta1, beta2, eps, weight_decay, step, loss_scale)


def adam_step_f64(master, m, v, g16, dtype, *, lr, beta1, beta2, eps, weight_decay, step,
                  loss_scale) -> None:
    """FP64 evaluation of the same update (error bound only), in place on float64 arrays."""
    _load().oracle_adam_step_f64(_ptr(master, np.float64), _ptr(m, np.float64),
                                 _ptr(v, np.float64), _ptr(g16, np.uint16), DTYPES[dtype],
                                 g16.size, float(np.float32(lr)), float(np.float32(beta1)),
                                 float(np.float32(beta2)), float(np.float32(eps)),
                                 float(np.float32(weight_decay)), step,
                                 float(np.float32(loss_scale)))


def grad_accumulate(acc, g16, dtype, first: bool) -> None:
    """acc = float(g16) if first else acc + float(g16), in FP32, in place."""
    if acc.size != g16.size:
        raise ValueError("length mismatch")
    _load().oracle_grad_accumulate(_ptr(acc, np.float32), _ptr(g16, np.uint16), DTYPES[dtype],
                                   g16.size, int(bool(first)))


def overflow_check_g32(g32, loss_scale: float) -> tuple[int, float]:
    """overflow_check over FP32 gradients: (found_inf, FP64 sum of unscaled squares)."""
    flag = np.zeros(1, np.int32)
    s = np.zeros(1, np.float64)
    _load().oracle_overflow_check_g32(_ptr(g32, np.float32), g32.size, loss_scale,
                                      flag.ctypes.data, s.ctypes.data)
    return int(flag[0]), float(s[0])


def adam_step_g32(w16, g32, master, m, v, dtype, *, lr, beta1, beta2, eps, weight_decay, step,
                  loss_scale) -> None:
    """adam_step with FP32 gradients (dtype is the working weights' format)."""
    count = g32.size
    for a in (w16, master, m, v):
        if a.size != count:
            raise ValueError("all shard arrays must have the same length")
    _load().oracle_adam_step_g32(_ptr(w16, np.uint16), _ptr(g32, np.float32),
                                 _ptr(master, np.float32), _ptr(m, np.float32),
                                 _ptr(v, np.float32), DTYPES[dtype], count, lr, beta1, beta2, eps,
                                 weight_decay, step, loss_scale)


FORMATS = {"f16": 0, "bf16": 1, "f32": 2}


def _ptr_array(arrays):
    arr = (ctypes.c_void_p * len(arrays))()
    for i, a in enumerate(arrays):
        if not a.flags.c_contiguous:
            raise ValueError("arrays must be C-contiguous")
        arr[i] = a.ctypes.data
    return arr


def reduce_shard(replicas, in_fmt: str, out_fmt: str, psi: int, n: int, rank: int) -> np.ndarray:
    """Rank `rank`'s chunk of the element-wise FP32 sum of n full replica buffers."""
    if len(replicas) != n:
        raise ValueError("one replica per rank")
    in_dt = np.float32 if in_fmt == "f32" else np.uint16
    for r in replicas:
        if r.dtype != in_dt or r.size < psi:
            raise ValueError("replica dtype or size")
    lay = layout(psi, n, rank)
    out = np.empty(lay.count, np.float32 if out_fmt == "f32" else np.uint16)
    _load().oracle_reduce_shard(out.ctypes.data, FORMATS[out_fmt], _ptr_array(replicas),
                                FORMATS[in_fmt], psi, n, rank)
    return out


def gather_shards(shards, psi: int, n: int, full: np.ndarray) -> np.ndarray:
    """Copy shard k (count_k elements) to full[k*S : k*S + count_k] for every rank k."""
    if len(shards) != n:
        raise ValueError("one shard per rank")
    for k, sh in enumerate(shards):
        if sh.dtype != full.dtype or sh.size < layout(psi, n, k).count:
            raise ValueError("shard dtype or size")
    _load().oracle_gather_shards(full.ctypes.data, _ptr_array(shards), full.itemsize, psi, n)
    return full


# ---------------------------------------------------------------------------
# Accounting the pages do in closed form (bytes and elements, integers).
# ---------------------------------------------------------------------------

def comm_volume(psi: int, n: int, stage: int, elem_bytes: int) -> dict:
    """Communication of one data-parallel step, per rank.

    elements: the pages' element count per rank per step -- 2 psi for plain
    data parallelism and ZeRO stages 1 and 2 (a reduce-scatter of psi and an
    all-gather of psi), 3 psi for stage 3 (a second all-gather) ("How far does
    splitting the batch get you?", "What does each stage cost on the wire?";
    "Stop Replicating What You Can Shard", FSDP communication equation).
    ring_bytes: what a ring actually sends per rank: each collective over an
    M-byte message sends (d-1)/d of it ("Why does the all-reduce not get more
    expensive with more ranks?"), with the message padded to n equal chunks.
    ring_hops: sequential hops of those collectives, 2(d-1) per all-reduce.
    """
    if stage not in (0, 1, 2, 3):
        raise ValueError("stage must be 0..3")
    lay = layout(psi, n, 0)
    collectives = 3 if stage == 3 else 2
    return {
        "collectives": collectives,
        "elements": collectives * psi,
        "wire_bytes": collectives * psi * elem_bytes,
        "ring_bytes": collectives * (n - 1) * lay.shard * elem_bytes,
        "ring_hops": collectives * (n - 1),
    }


def peak_memory(psi: int, n: int, unit_params: int, units_resident: int,
                activation_bytes: int) -> int:
    """ZeRO-3 peak per rank: the persistent 16 psi / N shard, plus the 16-bit
    weights of the units gathered at once, plus activations ("ZeRO Stage 3
    Math", "Peak transient memory")."""
    return layout(psi, n, 0).bytes_z3 + units_resident * unit_params * 2 + activation_bytes


@dataclass
class ScalerState:
    """Dynamic loss scale and applied-step counter held on the host."""
    loss_scale: float
    step: int = 0
    clean_steps: int = 0
    growth_interval: int = 2000


def policy(state: ScalerState, found_inf: int) -> bool:
    """Skip-or-apply decision after the overflow check ("Mixed-precision training").

    On overflow the step is skipped, the loss scale halves and the step counter
    stays.  Otherwise the counter advances (the update about to run is number
    ``state.step``) and, after ``growth_interval`` clean steps in a row, the
    scale doubles.  Returns True when the update must be applied.  An applied
    update unscales with the loss scale in force BEFORE this call (the one the
    gradients carry); ``state.loss_scale`` afterwards is the next step's.
    """
    S = np.float32(state.loss_scale)  # the scale is an FP32 number
    if found_inf:
        state.loss_scale = float(S / np.float32(2))
        state.clean_steps = 0
        return False
    state.step += 1
    state.clean_steps += 1
    if state.growth_interval and state.clean_steps >= state.growth_interval:
        with np.errstate(over="ignore"):
            grown = S * np.float32(2)
        if np.isfinite(grown):  # the scale stays a finite number
            state.loss_scale = float(grown)
        state.clean_steps = 0
    return True


# ---------------------------------------------------------------------------
# Parity bar: ordinal distance between bit patterns (test infrastructure).
# ---------------------------------------------------------------------------

def _ordinal(bits: np.ndarray, width: int) -> np.ndarray:
    """Map sign-magnitude float bit patterns onto a line where +0 and -0 meet."""
    b = bits.astype(np.int64)
    sign = np.int64(1) << (width - 1)
    mag = b & (sign - 1)
    return np.where(b & sign, -mag, mag)


def ulp_distance32(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """|ordinal(a) - ordinal(b)| for float32 arrays (NaN pairs count 0, NaN vs number huge)."""
    a = np.ascontiguousarray(a, np.float32)
    b = np.ascontiguousarray(b, np.float32)
    d = np.abs(_ordinal(a.view(np.uint32), 32) - _ordinal(b.view(np.uint32), 32))
    na, nb = np.isnan(a), np.isnan(b)
    d = np.where(na & nb, 0, d)
    return np.where(na ^ nb, np.int64(1) << 40, d)


def ulp_distance16(a: np.ndarray, b: np.ndarray, dtype: str) -> np.ndarray:
    """Same for 16-bit patterns of format dtype."""
    a = np.ascontiguousarray(a, np.uint16)
    b = np.ascontiguousarray(b, np.uint16)
    d = np.abs(_ordinal(a, 16) - _ordinal(b, 16))
    emask = 0x7C00 if dtype == "f16" else 0x7F80
    mmask = 0x03FF if dtype == "f16" else 0x007F
    na = ((a & emask) == emask) & ((a & mmask) != 0)
    nb = ((b & emask) == emask) & ((b & mmask) != 0)
    d = np.where(na & nb, 0, d)
    return np.where(na ^ nb, np.int64(1) << 40, d)


# ---------------------------------------------------------------------------
# Host-thread drivers.  The step is elementwise, so contiguous sub-ranges are
# independent; ctypes releases the GIL while the C loop runs.
# ---------------------------------------------------------------------------

def host_threads() -> int:
    """Threads to use on this host: its CPU share, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _ranges(count: int, threads: int):
    threads = max(1, min(threads, count // 4096 or 1))
    step = (count + threads - 1) // threads
    return [(s, min(count, s + step)) for s in range(0, count, step)]


def adam_step_mt(w16, g16, master, m, v, dtype, *, threads=None, **hp) -> int:
    """adam_step over sub-ranges on `threads` host threads; returns the threads used."""
    from concurrent.futures import ThreadPoolExecutor

    rs = _ranges(g16.size, threads or host_threads())
    with ThreadPoolExecutor(len(rs)) as ex:
        list(ex.map(lambda r: adam_step(w16[r[0]:r[1]], g16[r[0]:r[1]], master[r[0]:r[1]],
                                        m[r[0]:r[1]], v[r[0]:r[1]], dtype, **hp), rs))
    return len(rs)


def overflow_flag_mt(g16, dtype, loss_scale, threads=None) -> int:
    """The overflow flag of overflow_check, over sub-ranges on host threads."""
    from concurrent.futures import ThreadPoolExecutor

    rs = _ranges(g16.size, threads or host_threads())
    with ThreadPoolExecutor(len(rs)) as ex:
        flags = list(ex.map(lambda r: overflow_check(g16[r[0]:r[1]], dtype, loss_scale)[0], rs))
    return int(any(flags))
