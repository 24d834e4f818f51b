"""Python binding of libzero_shard.so, the ZeRO-sharded mixed-precision Adam step.

Argument marshalling only: tensors become device pointers, the stream
defaults to torch's current stream, and sizes are checked on the host before
anything is launched.  Every step of the computation runs in the library's
gfx950 kernels; there is no other code path.  Importing this package fails
loudly if the library has not been built.

Functions carry the names of the C entry points (include/zero_shard.h):

    zero_shard_layout(psi, n, rank) -> Layout
    zero_overflow_check(g16, psi, n, rank, loss_scale, found_inf, sumsq=None, partials=None)
    zero_adam_step(w16, g16, master, m, v, psi, n, rank, *, lr, beta1, beta2, eps,
                   weight_decay, step, loss_scale, found_inf=None)
    zero_scaler_update(state: Scaler, found_inf) -> bool   (skip-or-apply, loss scale)
    zero_strerror(code) -> str

and under short names: layout(psi, n, rank); overflow_check(g16, psi, n, rank,
loss_scale, found_inf, sumsq=None); adam_step(..., lr, betas=(b1, b2), eps,
weight_decay, step, loss_scale, found_inf=None).

FP32 gradients (accumulated across micro-batches):

    zero_grad_accumulate(acc32, g16, psi, n, rank, first)
    zero_grad_accumulate_check(acc32, g16, psi, n, rank, first, loss_scale, found_inf)  # last one
    zero_overflow_check_g32(g32, psi, n, rank, loss_scale, found_inf, sumsq=None, partials=None)
    zero_adam_step_g32(w16, g32, master, m, v, psi, n, rank, *, lr, ..., step, loss_scale)
    zero_overflow_check_g32_dev(g32, psi, n, rank, ctl)        # device-resident control
    zero_adam_step_g32_dev(w16, g32, master, m, v, psi, n, rank, lr=..., ..., ctl=ctl)

The exchanges around the step on one GPU, and their accounting:

    zero_reduce_shard(out, replicas, psi, n, rank)   # reduce-scatter result of one rank
    zero_gather_shards(full, shards, psi, n)          # all-gather into the flat buffer
    zero_comm_volume(psi, n, stage, elem_bytes) -> dict
    zero_peak_memory(psi, n, unit_params, units_resident, activation_bytes) -> int

Sharded checkpoints (host numpy arrays; one file per rank):

    zero_ckpt_write(path, psi, n, rank, dtype, scaler, w16, master, m, v)
    zero_ckpt_read_info(path) / zero_ckpt_verify(path) / zero_ckpt_read(path, first, count)
    zero_reshard_plan(psi, n_old, n_new, rank_new) -> [(src_rank, src_first, dst_first, count)]
    zero_ckpt_read_resharded(paths_old, psi, n_new, rank_new) -> (w16, master, m, v)

Device-resident control (no read-back between steps):

    ctl = device_ctl_new(loss_scale, device)            # zero_device_ctl in device memory
    bias = zero_bias_corrections(b1, b2, t_first, k).to(device)
    zero_overflow_check_dev(g16, psi, n, rank, ctl)
    zero_scaler_update_dev(ctl, bias, t_first)
    zero_adam_step_dev(w16, g16, master, m, v, psi, n, rank, lr=..., ..., ctl=ctl)
"""
from ._binding import (  # noqa: F401
    LIB_PATH,
    CkptInfo,
    SUMSQ_PARTIALS,
    DeviceCtl,
    Layout,
    Scaler,
    ZeroError,
    adam_step,
    layout,
    lib,
    overflow_check,
    device_ctl_new,
    device_ctl_read,
    zero_adam_step,
    zero_adam_step_dev,
    zero_adam_step_g32,
    zero_adam_step_g32_dev,
    zero_bias_corrections,
    zero_ckpt_read,
    zero_ckpt_read_info,
    zero_ckpt_read_resharded,
    zero_ckpt_verify,
    zero_ckpt_write,
    zero_comm_volume,
    zero_gather_shards,
    zero_grad_accumulate,
    zero_grad_accumulate_check,
    zero_grad_accumulate_check_dev,
    zero_overflow_check,
    zero_overflow_check_dev,
    zero_overflow_check_noalloc,
    zero_overflow_check_g32,
    zero_overflow_check_g32_dev,
    zero_peak_memory,
    zero_reduce_shard,
    zero_reduce_shard_check,
    zero_reduce_shard_check_dev,
    zero_reshard_plan,
    zero_scaler_update,
    zero_scaler_update_dev,
    zero_set_grid_cap,
    zero_set_occupancy,
    zero_set_launch_piece,
    zero_shard_layout,
    zero_strerror,
)

__all__ = [
    "Layout",
    "ZeroError",
    "zero_shard_layout",
    "zero_overflow_check",
    "zero_adam_step",
    "Scaler",
    "zero_scaler_update",
    "zero_strerror",
    "DeviceCtl",
    "device_ctl_new",
    "device_ctl_read",
    "zero_bias_corrections",
    "zero_overflow_check_dev",
    "zero_overflow_check_noalloc",
    "zero_scaler_update_dev",
    "zero_adam_step_dev",
    "zero_grad_accumulate",
    "zero_grad_accumulate_check",
    "zero_grad_accumulate_check_dev",
    "zero_overflow_check_g32",
    "zero_adam_step_g32",
    "zero_overflow_check_g32_dev",
    "zero_adam_step_g32_dev",
    "zero_reduce_shard",
    "zero_reduce_shard_check",
    "zero_reduce_shard_check_dev",
    "zero_gather_shards",
    "zero_comm_volume",
    "zero_peak_memory",
    "CkptInfo",
    "zero_ckpt_write",
    "zero_ckpt_read_info",
    "zero_ckpt_verify",
    "zero_ckpt_read",
    "zero_reshard_plan",
    "zero_ckpt_read_resharded",
    "zero_set_grid_cap",
    "zero_set_occupancy",
    "zero_set_launch_piece",
    "layout",
    "overflow_check",
    "adam_step",
]
