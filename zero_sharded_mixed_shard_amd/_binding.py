"""ctypes binding of libzero_shard.so (see include/zero_shard.h for the contract)."""
from __future__ import annotations

import ctypes
import functools
import os
from dataclasses import dataclass

import numpy as np
import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libzero_shard.so")
SUMSQ_PARTIALS = 4096  # ZERO_SUMSQ_PARTIALS

ZERO_F16, ZERO_BF16, ZERO_F32 = 0, 1, 2
MAX_LOCAL_RANKS = 64  # ZERO_MAX_LOCAL_RANKS
_DTYPES = {torch.float16: ZERO_F16, torch.bfloat16: ZERO_BF16}
_FORMATS = {torch.float16: ZERO_F16, torch.bfloat16: ZERO_BF16, torch.float32: ZERO_F32}


class ZeroError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {zero_strerror(code)} (code {code})")


if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python zero_sharded_mixed_shard_amd/build.py` "
        "(or __graft_entry__.build()); there is no fallback path")

lib = ctypes.CDLL(LIB_PATH)


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


_u64, _u32, _i32, _f32, _vp = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int, ctypes.c_float,
                               ctypes.c_void_p)
lib.zero_shard_layout.argtypes = [_u64, _u32, _u32, ctypes.POINTER(_Layout)]
lib.zero_shard_layout.restype = _i32
lib.zero_overflow_check.argtypes = [_vp, _i32, _u64, _u32, _u32, _f32, _vp, _vp, _vp, _vp]
lib.zero_overflow_check.restype = _i32
lib.zero_overflow_check_noalloc.argtypes = [_vp, _i32, _u64, _u32, _u32, _f32, _vp, _vp, _vp]
lib.zero_overflow_check_noalloc.restype = _i32
lib.zero_adam_step.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _u64, _u32, _u32, _f32, _f32, _f32,
                               _f32, _f32, _u64, _f32, _vp, _vp]
lib.zero_adam_step.restype = _i32


class Scaler(ctypes.Structure):
    """zero_scaler: dynamic loss scale and applied-update counter (host memory)."""
    _fields_ = [("loss_scale", ctypes.c_float), ("growth_interval", ctypes.c_uint32),
                ("step", ctypes.c_uint64), ("clean_steps", ctypes.c_uint64)]

    def __init__(self, loss_scale: float, growth_interval: int = 2000, step: int = 0):
        super().__init__(loss_scale, growth_interval, step, 0)


lib.zero_scaler_update.argtypes = [ctypes.POINTER(Scaler), ctypes.c_int32,
                                   ctypes.POINTER(ctypes.c_int32)]
lib.zero_scaler_update.restype = _i32


class DeviceCtl(ctypes.Structure):
    """zero_device_ctl: the control block the device-resident path keeps in device memory."""
    _fields_ = [("scaler", Scaler), ("found_inf", ctypes.c_int32), ("apply", ctypes.c_int32),
                ("loss_scale_used", ctypes.c_float), ("bc1", ctypes.c_float),
                ("bc2", ctypes.c_float), ("status", ctypes.c_int32),
                ("rcp_loss_scale", ctypes.c_double), ("rcp_bc1", ctypes.c_double),
                ("rcp_bc2", ctypes.c_double)]


lib.zero_grad_accumulate.argtypes = [_vp, _vp, _i32, _u64, _u32, _u32, ctypes.c_int32, _vp]
lib.zero_grad_accumulate_check.argtypes = [_vp, _vp, _i32, _u64, _u32, _u32, ctypes.c_int32,
                                           _f32, _vp, _vp]
lib.zero_grad_accumulate_check.restype = _i32
lib.zero_grad_accumulate_check_dev.argtypes = [_vp, _vp, _i32, _u64, _u32, _u32, ctypes.c_int32,
                                               _vp, _vp]
lib.zero_grad_accumulate_check_dev.restype = _i32
lib.zero_grad_accumulate.restype = _i32
lib.zero_overflow_check_g32.argtypes = [_vp, _u64, _u32, _u32, _f32, _vp, _vp, _vp, _vp]
lib.zero_overflow_check_g32.restype = _i32
lib.zero_adam_step_g32.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _u64, _u32, _u32, _f32, _f32,
                                   _f32, _f32, _f32, _u64, _f32, _vp, _vp]
lib.zero_adam_step_g32.restype = _i32
lib.zero_reduce_shard.argtypes = [_vp, _i32, _vp, _i32, _u64, _u32, _u32, _vp]
lib.zero_reduce_shard.restype = _i32
lib.zero_reduce_shard_check.argtypes = [_vp, _i32, _vp, _i32, _u64, _u32, _u32, _f32, _vp, _vp]
lib.zero_reduce_shard_check.restype = _i32
lib.zero_reduce_shard_check_dev.argtypes = [_vp, _i32, _vp, _i32, _u64, _u32, _u32, _vp, _vp]
lib.zero_reduce_shard_check_dev.restype = _i32
lib.zero_gather_shards.argtypes = [_vp, _vp, _i32, _u64, _u32, _vp]
lib.zero_gather_shards.restype = _i32


class _Comm(ctypes.Structure):
    _fields_ = [("collectives", ctypes.c_uint32), ("ring_hops", ctypes.c_uint32),
                ("elements", ctypes.c_uint64), ("wire_bytes", ctypes.c_uint64),
                ("ring_bytes", ctypes.c_uint64)]


lib.zero_comm_volume.argtypes = [_u64, _u32, _u32, _u32, ctypes.POINTER(_Comm)]
lib.zero_comm_volume.restype = _i32
lib.zero_peak_memory.argtypes = [_u64, _u32, _u64, _u32, _u64, ctypes.POINTER(ctypes.c_uint64)]
lib.zero_peak_memory.restype = _i32
lib.zero_bias_corrections.argtypes = [_f32, _f32, _u64, _u32, _vp]
lib.zero_bias_corrections.restype = _i32
lib.zero_overflow_check_dev.argtypes = [_vp, _i32, _u64, _u32, _u32, _vp, _vp]
lib.zero_overflow_check_dev.restype = _i32
lib.zero_scaler_update_dev.argtypes = [_vp, _vp, _u64, _u32, _vp]
lib.zero_scaler_update_dev.restype = _i32
lib.zero_adam_step_dev.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _u64, _u32, _u32, _f32, _f32,
                                   _f32, _f32, _f32, _vp, _vp]
lib.zero_adam_step_dev.restype = _i32
lib.zero_overflow_check_g32_dev.argtypes = [_vp, _u64, _u32, _u32, _vp, _vp]
lib.zero_overflow_check_g32_dev.restype = _i32
lib.zero_adam_step_g32_dev.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _u64, _u32, _u32, _f32,
                                       _f32, _f32, _f32, _f32, _vp, _vp]
lib.zero_adam_step_g32_dev.restype = _i32
lib.zero_set_grid_cap.argtypes = [_u32]
lib.zero_set_occupancy.argtypes = [_u32]
lib.zero_set_occupancy.restype = _i32
lib.zero_set_grid_cap.restype = _i32
lib.zero_set_launch_piece.argtypes = [_u64]
lib.zero_set_launch_piece.restype = _i32
lib.zero_strerror.argtypes = [_i32]
lib.zero_strerror.restype = ctypes.c_char_p


def zero_strerror(code: int) -> str:
    return lib.zero_strerror(code).decode()


def zero_set_grid_cap(blocks: int) -> None:
    """Cap every streaming kernel's grid at `blocks` workgroups (0 restores the default)."""
    if not 0 <= blocks < 1 << 32:
        raise ValueError("blocks must fit in 32 bits")
    lib.zero_set_grid_cap(blocks)


def zero_set_occupancy(blocks_per_cu: int) -> None:
    """Resident blocks per CU of this thread's streaming-kernel launches (step, accumulates,
    flag-only check, reduce and gather): 0 leaves each kernel its own rule, 1-7 cap, 8+ removes
    the cap."""
    if not 0 <= blocks_per_cu < 1 << 32:
        raise ValueError("blocks_per_cu must fit in 32 bits")
    lib.zero_set_occupancy(blocks_per_cu)


def zero_set_launch_piece(elements: int) -> None:
    """Most elements per launch of this thread's step, accumulate and flag-only check launches;
    a longer shard goes out as consecutive launches on one stream.  0 restores each kernel's
    rule (the step and the fused-check accumulate of a later micro-batch: launches of 2^27 once
    a shard holds two; the other accumulates and the check: one launch); 2**64 - 1 means one
    launch."""
    if not 0 <= elements < 1 << 64:
        raise ValueError("elements must fit in 64 bits")
    lib.zero_set_launch_piece(elements)


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


@functools.lru_cache(maxsize=4096)
def zero_shard_layout(psi: int, n: int, rank: int) -> Layout:
    """The layout of (psi, n, rank); results are cached (Layout is immutable)."""
    out = _Layout()
    rc = lib.zero_shard_layout(psi, n, rank, ctypes.byref(out))
    if rc != 0:
        raise ZeroError(rc, "zero_shard_layout")
    return Layout(*(getattr(out, f) for f, _ in _Layout._fields_))


_raw_current_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_handle(stream, device) -> int:
    """hipStream_t of `stream`, or of torch's current stream on `device`."""
    if stream is None:
        if _raw_current_stream is not None:
            return int(_raw_current_stream(device.index if device.index is not None
                                           else torch.cuda.current_device()))
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _view(t: torch.Tensor, name: str, dtypes, count: int, device) -> int:
    """Pointer of a 1-D contiguous device tensor holding at least `count` elements."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device}): the kernels "
                         "read and write device memory only")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {list(dtypes)}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dim() != 1 or not t.is_contiguous():
        raise ValueError(f"{name} must be a 1-D contiguous view")
    if t.numel() < count:
        raise ValueError(f"{name} holds {t.numel()} elements, the shard needs {count}")
    return t.data_ptr()


def zero_overflow_check(g16: torch.Tensor, psi: int, n: int, rank: int, loss_scale: float,
                        found_inf: torch.Tensor, sumsq: torch.Tensor | None = None,
                        partials: torch.Tensor | None = None, stream=None) -> None:
    """Unscale this rank's gradients by loss_scale; found_inf[0] := 1 iff any is inf/NaN."""
    lay = zero_shard_layout(psi, n, rank)
    dev = g16.device
    if dev.type != "cuda":
        raise ValueError("g16 must be a device tensor")
    p_g = _view(g16, "g16", _DTYPES, lay.count, dev)
    p_f = _view(found_inf, "found_inf", (torch.int32,), 1, dev)
    p_s = p_p = None
    if sumsq is not None:
        p_s = _view(sumsq, "sumsq", (torch.float32,), 1, dev)
        if partials is None:
            raise ValueError("sumsq needs a partials buffer of SUMSQ_PARTIALS float64")
        p_p = _view(partials, "partials", (torch.float64,), SUMSQ_PARTIALS, dev)
    with torch.cuda.device(dev):
        rc = lib.zero_overflow_check(p_g, _DTYPES[g16.dtype], psi, n, rank, loss_scale, p_f, p_s,
                                     p_p, _stream_handle(stream, dev))
    if rc != 0:
        raise ZeroError(rc, "zero_overflow_check")


def zero_overflow_check_noalloc(g16: torch.Tensor, psi: int, n: int, rank: int,
                                loss_scale: float, found_inf: torch.Tensor,
                                sumsq: torch.Tensor | None = None, stream=None) -> None:
    """zero_overflow_check with the library's fixed per-device partials (no workspace)."""
    lay = zero_shard_layout(psi, n, rank)
    dev = g16.device
    if dev.type != "cuda":
        raise ValueError("g16 must be a device tensor")
    p_g = _view(g16, "g16", _DTYPES, lay.count, dev)
    p_f = _view(found_inf, "found_inf", (torch.int32,), 1, dev)
    p_s = _view(sumsq, "sumsq", (torch.float32,), 1, dev) if sumsq is not None else None
    with torch.cuda.device(dev):
        rc = lib.zero_overflow_check_noalloc(p_g, _DTYPES[g16.dtype], psi, n, rank, loss_scale,
                                             p_f, p_s, _stream_handle(stream, dev))
    if rc != 0:
        raise ZeroError(rc, "zero_overflow_check_noalloc")


def zero_adam_step(w16: torch.Tensor, g16: torch.Tensor, master: torch.Tensor, m: torch.Tensor,
                   v: torch.Tensor, psi: int, n: int, rank: int, *, lr: float, beta1: float,
                   beta2: float, eps: float, weight_decay: float, step: int, loss_scale: float,
                   found_inf: torch.Tensor | None = None, stream=None) -> None:
    """One Adam/AdamW step over rank `rank`'s shard; every array is a shard view."""
    lay = zero_shard_layout(psi, n, rank)
    dev = g16.device
    if dev.type != "cuda":
        raise ValueError("g16 must be a device tensor")
    if w16.dtype != g16.dtype:
        raise TypeError("w16 and g16 must share one 16-bit dtype")
    ptrs = [
        _view(w16, "w16", _DTYPES, lay.count, dev),
        _view(g16, "g16", _DTYPES, lay.count, dev),
        _view(master, "master", (torch.float32,), lay.count, dev),
        _view(m, "m", (torch.float32,), lay.count, dev),
        _view(v, "v", (torch.float32,), lay.count, dev),
    ]
    p_f = None if found_inf is None else _view(found_inf, "found_inf", (torch.int32,), 1, dev)
    with torch.cuda.device(dev):
        rc = lib.zero_adam_step(*ptrs, _DTYPES[g16.dtype], psi, n, rank, lr, beta1, beta2, eps,
                                weight_decay, step, loss_scale, p_f, _stream_handle(stream, dev))
    if rc != 0:
        raise ZeroError(rc, "zero_adam_step")


# ---- short names of the three path calls ----------------------------------------

def layout(psi: int, n: int, rank: int) -> Layout:
    """zero_shard_layout under its short name."""
    return zero_shard_layout(psi, n, rank)


def overflow_check(g16: torch.Tensor, psi: int, n: int, rank: int, loss_scale: float,
                   found_inf: torch.Tensor, sumsq: torch.Tensor | None = None,
                   partials: torch.Tensor | None = None, stream=None) -> None:
    """zero_overflow_check under its short name; with `sumsq` and no `partials`, the
    partial-sum buffer is taken from torch's allocator for this call."""
    if sumsq is not None and partials is None:
        partials = torch.empty(SUMSQ_PARTIALS, dtype=torch.float64, device=g16.device)
    zero_overflow_check(g16, psi, n, rank, loss_scale, found_inf, sumsq, partials, stream)


def adam_step(w16: torch.Tensor, g16: torch.Tensor, master: torch.Tensor, m: torch.Tensor,
              v: torch.Tensor, psi: int, n: int, rank: int, *, lr: float, betas, eps: float,
              weight_decay: float, step: int, loss_scale: float,
              found_inf: torch.Tensor | None = None, stream=None) -> None:
    """zero_adam_step under its short name, with the two betas as one pair."""
    beta1, beta2 = betas
    zero_adam_step(w16, g16, master, m, v, psi, n, rank, lr=lr, beta1=beta1, beta2=beta2,
                   eps=eps, weight_decay=weight_decay, step=step, loss_scale=loss_scale,
                   found_inf=found_inf, stream=stream)


def zero_scaler_update(state: Scaler, found_inf: int) -> bool:
    """Skip-or-apply decision; returns True when the update must run (see the header)."""
    apply = ctypes.c_int32(0)
    rc = lib.zero_scaler_update(ctypes.byref(state), int(found_inf), ctypes.byref(apply))
    if rc != 0:
        raise ZeroError(rc, "zero_scaler_update")
    return bool(apply.value)


# ---- device-resident control -------------------------------------------------

def device_ctl_new(loss_scale: float, device, growth_interval: int = 2000,
                   step: int = 0) -> torch.Tensor:
    """A zero_device_ctl in device memory (a uint8 tensor), initialised from the host."""
    host = DeviceCtl()
    host.scaler = Scaler(loss_scale, growth_interval, step)
    raw = torch.frombuffer(bytearray(bytes(host)), dtype=torch.uint8)
    return raw.to(device)


def device_ctl_read(ctl: torch.Tensor) -> DeviceCtl:
    """Copy a device control block back to the host (synchronises the stream)."""
    return DeviceCtl.from_buffer_copy(bytes(ctl.cpu().numpy().tobytes()))


def _ctl_ptr(ctl: torch.Tensor, device) -> int:
    if ctl.dtype != torch.uint8 or ctl.numel() < ctypes.sizeof(DeviceCtl) or \
            ctl.device != device or ctl.device.type != "cuda" or not ctl.is_contiguous():
        raise ValueError(f"ctl must be a contiguous uint8 device tensor of "
                         f"{ctypes.sizeof(DeviceCtl)} bytes on {device}")
    return ctl.data_ptr()


def zero_bias_corrections(beta1: float, beta2: float, t_first: int, length: int) -> torch.Tensor:
    """Host table [bc1 of t_first .. t_first+length-1, then bc2 of the same t] (float32)."""
    out = torch.empty(2 * length, dtype=torch.float32)
    rc = lib.zero_bias_corrections(beta1, beta2, t_first, length, out.data_ptr())
    if rc != 0:
        raise ZeroError(rc, "zero_bias_corrections")
    return out


def zero_overflow_check_dev(g16: torch.Tensor, psi: int, n: int, rank: int, ctl: torch.Tensor,
                            stream=None) -> None:
    """Overflow check with S read on the device; writes ctl.found_inf."""
    lay = zero_shard_layout(psi, n, rank)
    dev = g16.device
    p_g = _view(g16, "g16", _DTYPES, lay.count, dev)
    with torch.cuda.device(dev):
        rc = lib.zero_overflow_check_dev(p_g, _DTYPES[g16.dtype], psi, n, rank,
                                         _ctl_ptr(ctl, dev), _stream_handle(stream, dev))
    if rc != 0:
        raise ZeroError(rc, "zero_overflow_check_dev")


def zero_scaler_update_dev(ctl: torch.Tensor, bias: torch.Tensor, t_first: int,
                           stream=None) -> None:
    """Skip-or-apply decision on the device; `bias` is a device copy of zero_bias_corrections."""
    dev = ctl.device
    if bias.dtype != torch.float32 or bias.device != dev or dev.type != "cuda" or \
            bias.dim() != 1 or bias.numel() % 2 or not bias.is_contiguous():
        raise ValueError("bias must be a 1-D float32 device tensor of 2*length entries")
    with torch.cuda.device(dev):
        rc = lib.zero_scaler_update_dev(_ctl_ptr(ctl, dev), bias.data_ptr(), t_first,
                                        bias.numel() // 2, _stream_handle(stream, dev))
    if rc != 0:
        raise ZeroError(rc, "zero_scaler_update_dev")


def zero_adam_step_dev(w16: torch.Tensor, g16: torch.Tensor, master: torch.Tensor,
                       m: torch.Tensor, v: torch.Tensor, psi: int, n: int, rank: int, *,
                       lr: float, beta1: float, beta2: float, eps: float, weight_decay: float,
                       ctl: torch.Tensor, stream=None) -> None:
    """Adam step with S and the bias corrections read from the device control block."""
    lay = zero_shard_layout(psi, n, rank)
    dev = g16.device
    if w16.dtype != g16.dtype:
        raise TypeError("w16 and g16 must share one 16-bit dtype")
    ptrs = [
        _view(w16, "w16", _DTYPES, lay.count, dev),
        _view(g16, "g16", _DTYPES, lay.count, dev),
        _view(master, "master", (torch.float32,), lay.count, dev),
        _view(m, "m", (torch.float32,), lay.count, dev),
        _view(v, "v", (torch.float32,), lay.count, dev),
    ]
    with torch.cuda.device(dev):
        rc = lib.zero_adam_step_dev(*ptrs, _DTYPES[g16.dtype], psi, n, rank, lr, beta1, beta2,
                                    eps, weight_decay, _ctl_ptr(ctl, dev),
                                    _stream_handle(stream, dev))
    if rc != 0:
        raise ZeroError(rc, "zero_adam_step_dev")


# ---- FP32 gradients ------------------------------------------------------------

def zero_grad_accumulate(acc: torch.Tensor, g16: torch.Tensor, psi: int, n: int, rank: int,
                         first: bool, stream=None) -> None:
    """acc = float(g16) (first) or acc + float(g16): one micro-batch into the FP32 accumulator."""
    lay = zero_shard_layout(psi, n, rank)
    dev = g16.device
    p_g = _view(g16, "g16", _DTYPES, lay.count, dev)
    p_a = _view(acc, "acc", (torch.float32,), lay.count, dev)
    with torch.cuda.device(dev):
        rc = lib.zero_grad_accumulate(p_a, p_g, _DTYPES[g16.dtype], psi, n, rank, int(bool(first)),
                                      _stream_handle(stream, dev))
    if rc != 0:
        raise ZeroError(rc, "zero_grad_accumulate")


def zero_grad_accumulate_check(acc: torch.Tensor, g16: torch.Tensor, psi: int, n: int,
                               rank: int, first: bool, loss_scale: float, found_inf: torch.Tensor,
                               stream=None) -> None:
    """The last micro-batch's accumulate with the FP32 overflow check of the result fused in."""
    lay = zero_shard_layout(psi, n, rank)
    dev = g16.device
    p_g = _view(g16, "g16", _DTYPES, lay.count, dev)
    p_a = _view(acc, "acc", (torch.float32,), lay.count, dev)
    p_f = _view(found_inf, "found_inf", (torch.int32,), 1, dev)
    with torch.cuda.device(dev):
        rc = lib.zero_grad_accumulate_check(p_a, p_g, _DTYPES[g16.dtype], psi, n, rank,
                                            int(bool(first)), loss_scale, p_f,
                                            _stream_handle(stream, dev))
    if rc != 0:
        raise ZeroError(rc, "zero_grad_accumulate_check")


def zero_grad_accumulate_check_dev(acc: torch.Tensor, g16: torch.Tensor, psi: int, n: int,
                                   rank: int, first: bool, ctl: torch.Tensor,
                                   stream=None) -> None:
    """zero_grad_accumulate_check with S read from, and the flag written to, the control block."""
    lay = zero_shard_layout(psi, n, rank)
    dev = g16.device
    p_g = _view(g16, "g16", _DTYPES, lay.count, dev)
    p_a = _view(acc, "acc", (torch.float32,), lay.count, dev)
    with torch.cuda.device(dev):
        rc = lib.zero_grad_accumulate_check_dev(p_a, p_g, _DTYPES[g16.dtype], psi, n, rank,
                                                int(bool(first)), _ctl_ptr(ctl, dev),
                                                _stream_handle(stream, dev))
    if rc != 0:
        raise ZeroError(rc, "zero_grad_accumulate_check_dev")


def zero_overflow_check_g32(g32: torch.Tensor, psi: int, n: int, rank: int, loss_scale: float,
                            found_inf: torch.Tensor, sumsq: torch.Tensor | None = None,
                            partials: torch.Tensor | None = None, stream=None) -> None:
    """Overflow check (and optional sum of squares) over FP32 gradients."""
    lay = zero_shard_layout(psi, n, rank)
    dev = g32.device
    p_g = _view(g32, "g32", (torch.float32,), lay.count, dev)
    p_f = _view(found_inf, "found_inf", (torch.int32,), 1, dev)
    p_s = p_p = None
    if sumsq is not None:
        p_s = _view(sumsq, "sumsq", (torch.float32,), 1, dev)
        if partials is None:
            raise ValueError("sumsq needs a partials buffer of SUMSQ_PARTIALS float64")
        p_p = _view(partials, "partials", (torch.float64,), SUMSQ_PARTIALS, dev)
    with torch.cuda.device(dev):
        rc = lib.zero_overflow_check_g32(p_g, psi, n, rank, loss_scale, p_f, p_s, p_p,
                                         _stream_handle(stream, dev))
    if rc != 0:
        raise ZeroError(rc, "zero_overflow_check_g32")


def zero_adam_step_g32(w16: torch.Tensor, g32: torch.Tensor, master: torch.Tensor,
                       m: torch.Tensor, v: torch.Tensor, psi: int, n: int, rank: int, *,
                       lr: float, beta1: float, beta2: float, eps: float, weight_decay: float,
                       step: int, loss_scale: float, found_inf: torch.Tensor | None = None,
                       stream=None) -> None:
    """Adam step reading FP32 gradients; w16's dtype sets the working weights' format."""
    lay = zero_shard_layout(psi, n, rank)
    dev = g32.device
    ptrs = [
        _view(w16, "w16", _DTYPES, lay.count, dev),
        _view(g32, "g32", (torch.float32,), lay.count, dev),
        _view(master, "master", (torch.float32,), lay.count, dev),
        _view(m, "m", (torch.float32,), lay.count, dev),
        _view(v, "v", (torch.float32,), lay.count, dev),
    ]
    p_f = None if found_inf is None else _view(found_inf, "found_inf", (torch.int32,), 1, dev)
    with torch.cuda.device(dev):
        rc = lib.zero_adam_step_g32(*ptrs, _DTYPES[w16.dtype], psi, n, rank, lr, beta1, beta2,
                                    eps, weight_decay, step, loss_scale, p_f,
                                    _stream_handle(stream, dev))
    if rc != 0:
        raise ZeroError(rc, "zero_adam_step_g32")


def zero_overflow_check_g32_dev(g32: torch.Tensor, psi: int, n: int, rank: int,
                                ctl: torch.Tensor, stream=None) -> None:
    """Overflow check of FP32 gradients with S read on the device; writes ctl.found_inf."""
    lay = zero_shard_layout(psi, n, rank)
    dev = g32.device
    p_g = _view(g32, "g32", (torch.float32,), lay.count, dev)
    with torch.cuda.device(dev):
        rc = lib.zero_overflow_check_g32_dev(p_g, psi, n, rank, _ctl_ptr(ctl, dev),
                                             _stream_handle(stream, dev))
    if rc != 0:
        raise ZeroError(rc, "zero_overflow_check_g32_dev")


def zero_adam_step_g32_dev(w16: torch.Tensor, g32: torch.Tensor, master: torch.Tensor,
                           m: torch.Tensor, v: torch.Tensor, psi: int, n: int, rank: int, *,
                           lr: float, beta1: float, beta2: float, eps: float,
                           weight_decay: float, ctl: torch.Tensor, stream=None) -> None:
    """Adam step on FP32 gradients with S and the bias corrections read from the control block."""
    lay = zero_shard_layout(psi, n, rank)
    dev = g32.device
    ptrs = [
        _view(w16, "w16", _DTYPES, lay.count, dev),
        _view(g32, "g32", (torch.float32,), lay.count, dev),
        _view(master, "master", (torch.float32,), lay.count, dev),
        _view(m, "m", (torch.float32,), lay.count, dev),
        _view(v, "v", (torch.float32,), lay.count, dev),
    ]
    with torch.cuda.device(dev):
        rc = lib.zero_adam_step_g32_dev(*ptrs, _DTYPES[w16.dtype], psi, n, rank, lr, beta1,
                                        beta2, eps, weight_decay, _ctl_ptr(ctl, dev),
                                        _stream_handle(stream, dev))
    if rc != 0:
        raise ZeroError(rc, "zero_adam_step_g32_dev")


# ---- exchanges on one GPU and accounting ------------------------------------------

def _ptr_list(tensors):
    arr = (ctypes.c_void_p * len(tensors))()
    for i, t in enumerate(tensors):
        arr[i] = None if t is None else t.data_ptr()
    return arr


def zero_reduce_shard(out: torch.Tensor, replicas, psi: int, n: int, rank: int,
                      stream=None) -> None:
    """Rank `rank`'s chunk of the FP32 sum of n full replica buffers, written in out's format."""
    lay = zero_shard_layout(psi, n, rank)
    dev = out.device
    if len(replicas) != n:
        raise ValueError(f"need {n} replicas, got {len(replicas)}")
    in_dt = replicas[0].dtype
    for k, r in enumerate(replicas):
        _view(r, f"replica {k}", (in_dt,), psi, dev)
    if in_dt not in _FORMATS:
        raise TypeError(f"replica dtype {in_dt} not supported")
    p_out = _view(out, "out", tuple(_FORMATS), lay.count, dev)
    with torch.cuda.device(dev):
        rc = lib.zero_reduce_shard(p_out, _FORMATS[out.dtype], _ptr_list(replicas),
                                   _FORMATS[in_dt], psi, n, rank, _stream_handle(stream, dev))
    if rc != 0:
        raise ZeroError(rc, "zero_reduce_shard")


def _reduce_views(out, replicas, psi, n, rank):
    lay = zero_shard_layout(psi, n, rank)
    dev = out.device
    if len(replicas) != n:
        raise ValueError(f"need {n} replicas, got {len(replicas)}")
    in_dt = replicas[0].dtype
    for k, r in enumerate(replicas):
        _view(r, f"replica {k}", (in_dt,), psi, dev)
    if in_dt not in _FORMATS:
        raise TypeError(f"replica dtype {in_dt} not supported")
    p_out = _view(out, "out", tuple(_FORMATS), lay.count, dev)
    return dev, in_dt, p_out


def zero_reduce_shard_check(out: torch.Tensor, replicas, psi: int, n: int, rank: int,
                            loss_scale: float, found_inf: torch.Tensor, stream=None) -> None:
    """zero_reduce_shard with the overflow check of the written chunk fused in: found_inf
    becomes 1 iff some out[i] / loss_scale is not finite."""
    dev, in_dt, p_out = _reduce_views(out, replicas, psi, n, rank)
    p_f = _view(found_inf, "found_inf", (torch.int32,), 1, dev)
    with torch.cuda.device(dev):
        rc = lib.zero_reduce_shard_check(p_out, _FORMATS[out.dtype], _ptr_list(replicas),
                                         _FORMATS[in_dt], psi, n, rank, loss_scale, p_f,
                                         _stream_handle(stream, dev))
    if rc != 0:
        raise ZeroError(rc, "zero_reduce_shard_check")


def zero_reduce_shard_check_dev(out: torch.Tensor, replicas, psi: int, n: int, rank: int,
                                ctl: torch.Tensor, stream=None) -> None:
    """zero_reduce_shard_check with S read from, and the flag written to, the control block."""
    dev, in_dt, p_out = _reduce_views(out, replicas, psi, n, rank)
    with torch.cuda.device(dev):
        rc = lib.zero_reduce_shard_check_dev(p_out, _FORMATS[out.dtype], _ptr_list(replicas),
                                             _FORMATS[in_dt], psi, n, rank, _ctl_ptr(ctl, dev),
                                             _stream_handle(stream, dev))
    if rc != 0:
        raise ZeroError(rc, "zero_reduce_shard_check_dev")


def zero_gather_shards(full: torch.Tensor, shards, psi: int, n: int, stream=None) -> None:
    """full[k*S : k*S + count_k] = shards[k] for every rank k (all-gather semantics)."""
    dev = full.device
    if len(shards) != n:
        raise ValueError(f"need {n} shards, got {len(shards)}")
    p_full = _view(full, "full", tuple(_FORMATS), psi, dev)
    for k, sh in enumerate(shards):
        cnt = zero_shard_layout(psi, n, k).count
        if sh is None:
            if cnt:
                raise ValueError(f"shard {k} holds {cnt} elements and cannot be None")
            continue
        _view(sh, f"shard {k}", (full.dtype,), cnt, dev)
    with torch.cuda.device(dev):
        rc = lib.zero_gather_shards(p_full, _ptr_list(shards), _FORMATS[full.dtype], psi, n,
                                    _stream_handle(stream, dev))
    if rc != 0:
        raise ZeroError(rc, "zero_gather_shards")


def zero_comm_volume(psi: int, n: int, stage: int, elem_bytes: int) -> dict:
    out = _Comm()
    rc = lib.zero_comm_volume(psi, n, stage, elem_bytes, ctypes.byref(out))
    if rc != 0:
        raise ZeroError(rc, "zero_comm_volume")
    return {f: getattr(out, f) for f, _ in _Comm._fields_}


def zero_peak_memory(psi: int, n: int, unit_params: int, units_resident: int,
                     activation_bytes: int) -> int:
    out = ctypes.c_uint64(0)
    rc = lib.zero_peak_memory(psi, n, unit_params, units_resident, activation_bytes,
                              ctypes.byref(out))
    if rc != 0:
        raise ZeroError(rc, "zero_peak_memory")
    return out.value


# ---- sharded checkpoints (host arrays) ---------------------------------------------

class CkptInfo(ctypes.Structure):
    """zero_ckpt_info."""
    _fields_ = [("psi", ctypes.c_uint64), ("n", ctypes.c_uint32), ("rank", ctypes.c_uint32),
                ("offset", ctypes.c_uint64), ("count", ctypes.c_uint64), ("dtype", ctypes.c_int),
                ("scaler", Scaler)]


class _Piece(ctypes.Structure):
    _fields_ = [("src_rank", ctypes.c_uint32), ("src_first", ctypes.c_uint64),
                ("dst_first", ctypes.c_uint64), ("count", ctypes.c_uint64)]


_cp = ctypes.c_char_p
lib.zero_ckpt_write.argtypes = [_cp, ctypes.POINTER(CkptInfo), _vp, _vp, _vp, _vp]
lib.zero_ckpt_read_info.argtypes = [_cp, ctypes.POINTER(CkptInfo)]
lib.zero_ckpt_verify.argtypes = [_cp]
lib.zero_ckpt_read.argtypes = [_cp, _u64, _u64, _vp, _vp, _vp, _vp]
lib.zero_reshard_plan.argtypes = [_u64, _u32, _u32, _u32, ctypes.POINTER(_Piece), _u32,
                                  ctypes.POINTER(ctypes.c_uint32)]
lib.zero_ckpt_read_resharded.argtypes = [_vp, _u32, _u64, _u32, _u32, _vp, _vp, _vp, _vp]
for _f in ("zero_ckpt_write", "zero_ckpt_read_info", "zero_ckpt_verify", "zero_ckpt_read",
           "zero_reshard_plan", "zero_ckpt_read_resharded"):
    getattr(lib, _f).restype = _i32

_DTYPE_CODES = {"f16": ZERO_F16, "bf16": ZERO_BF16, torch.float16: ZERO_F16,
                torch.bfloat16: ZERO_BF16}


def _host(a: np.ndarray, dtype, count: int, name: str) -> int:
    if not isinstance(a, np.ndarray) or a.dtype != dtype or not a.flags.c_contiguous:
        raise TypeError(f"{name} must be a C-contiguous numpy {np.dtype(dtype)} array")
    if a.size < count:
        raise ValueError(f"{name} holds {a.size} elements, the shard needs {count}")
    return a.ctypes.data


def zero_ckpt_write(path: str, psi: int, n: int, rank: int, dtype, scaler: Scaler,
                    w16: np.ndarray, master: np.ndarray, m: np.ndarray, v: np.ndarray) -> None:
    """Write one rank's slice (host numpy arrays: uint16 bit patterns and float32)."""
    cnt = zero_shard_layout(psi, n, rank).count
    info = CkptInfo(psi, n, rank, 0, 0, _DTYPE_CODES[dtype], scaler)
    rc = lib.zero_ckpt_write(os.fsencode(path), ctypes.byref(info),
                             _host(w16, np.uint16, cnt, "w16"), _host(master, np.float32, cnt, "master"),
                             _host(m, np.float32, cnt, "m"), _host(v, np.float32, cnt, "v"))
    if rc != 0:
        raise ZeroError(rc, "zero_ckpt_write")


def zero_ckpt_read_info(path: str) -> CkptInfo:
    info = CkptInfo()
    rc = lib.zero_ckpt_read_info(os.fsencode(path), ctypes.byref(info))
    if rc != 0:
        raise ZeroError(rc, "zero_ckpt_read_info")
    return info


def zero_ckpt_verify(path: str) -> None:
    rc = lib.zero_ckpt_verify(os.fsencode(path))
    if rc != 0:
        raise ZeroError(rc, "zero_ckpt_verify")


def zero_ckpt_read(path: str, first: int, count: int):
    """Elements [first, first + count) of a shard file: (w16 uint16, master, m, v float32)."""
    out = (np.empty(count, np.uint16), np.empty(count, np.float32), np.empty(count, np.float32),
           np.empty(count, np.float32))
    rc = lib.zero_ckpt_read(os.fsencode(path), first, count, *(a.ctypes.data for a in out))
    if rc != 0:
        raise ZeroError(rc, "zero_ckpt_read")
    return out


def zero_reshard_plan(psi: int, n_old: int, n_new: int, rank_new: int) -> list:
    """[(src_rank, src_first, dst_first, count), ...] for rank_new of the new layout."""
    cnt = ctypes.c_uint32(0)
    rc = lib.zero_reshard_plan(psi, n_old, n_new, rank_new, None, 0, ctypes.byref(cnt))
    if rc != 0:
        raise ZeroError(rc, "zero_reshard_plan")
    pieces = (_Piece * max(1, cnt.value))()
    rc = lib.zero_reshard_plan(psi, n_old, n_new, rank_new, pieces, cnt.value, ctypes.byref(cnt))
    if rc != 0:
        raise ZeroError(rc, "zero_reshard_plan")
    return [(p.src_rank, p.src_first, p.dst_first, p.count) for p in pieces[:cnt.value]]


def zero_ckpt_read_resharded(paths_old, psi: int, n_new: int, rank_new: int):
    """Rank rank_new's slice of an n_new-rank layout from the old shard files."""
    cnt = zero_shard_layout(psi, n_new, rank_new).count
    out = (np.empty(cnt, np.uint16), np.empty(cnt, np.float32), np.empty(cnt, np.float32),
           np.empty(cnt, np.float32))
    arr = (ctypes.c_char_p * len(paths_old))(*[os.fsencode(p) for p in paths_old])
    rc = lib.zero_ckpt_read_resharded(ctypes.cast(arr, ctypes.c_void_p), len(paths_old), psi,
                                      n_new, rank_new, *(a.ctypes.data for a in out))
    if rc != 0:
        raise ZeroError(rc, "zero_ckpt_read_resharded")
    return out
