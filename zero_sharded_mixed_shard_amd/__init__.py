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
"""
from ._binding import (  # noqa: F401
    LIB_PATH,
    SUMSQ_PARTIALS,
    Layout,
    Scaler,
    ZeroError,
    lib,
    zero_adam_step,
    zero_overflow_check,
    zero_scaler_update,
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
]
