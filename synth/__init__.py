"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module only draws random numbers and describes workloads; it holds none
of the optimizer's arithmetic.  Both the tests and the benchmark take their
inputs from here, so the oracle and the HIP library see identical bytes.

Workloads (the pages print no training data; every input is synthetic):

* ``C1``  flat buffer of 1,000,000 params, N = 8, rank 3; FP16 grads ~N(0,1e-3),
  FP32 master ~N(0,0.02), m = v = 0; Adam lr 1e-3, betas (0.9, 0.999),
  eps 1e-8, wd 0, loss scale 1; 3 steps.
* ``C2``  a flat buffer with GPT-2-small's 148 tensor shapes (124,439,808 params),
  N = 8; FP16 grads ~N(0,1e-3), loss scale 1024; AdamW wd 0.01; 10 steps.
* ``C3``  7.5e9 params, N = 8 (937.5M per shard); BF16 grads ~N(0,1e-4),
  moments drawn as if warm-started by 100 steps; AdamW lr 3e-4, wd 0.01; 20 steps.
* ``C4``  1e10 params, N = 1 (the 160 GB unsharded case); FP16 grads ~N(0,1e-3),
  loss scale 65536; AdamW lr 1e-4, wd 0.1; 5 steps.
* ``C5``  8,810,000,003 params, N = 64, rank 63 (ragged tail, 61 padding
  elements, shard start = 5 mod 8); FP16 grads with one entry in 1e7 set to
  +-inf/NaN on alternate steps; Adam, loss scale 65536 halving on overflow; 10 steps.

The sizes mirror the pages' worked examples: 7.5B ("ZeRO memory math",
worked example), 10B ("ZeRO Stage 3 Math", "A worked memory example") and
8.81B per data-parallel rank at d = 64 ("How far does splitting the batch get
you?").
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

CHUNK = 1 << 26  # elements per generation chunk on large buffers


def seed_of(cfg: int, buf: int, step: int = 0) -> int:
    """Seed convention: 1000*config + 100*buffer + step.

    Buffers: 1 = gradients, 2 = master, 3 = m, 4 = v, 5 = non-finite injection.
    """
    return 1000 * cfg + 100 * buf + step


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def fill_normal_(t: torch.Tensor, std: float, seed: int) -> torch.Tensor:
    """Fill a 1-D tensor (fp32, fp16 or bf16) in place with N(0, std^2) draws.

    Draws are made in FP32 chunk by chunk and stored with the tensor's dtype,
    so a 16-bit tensor holds the 16-bit value nearest to each draw.
    """
    g = _gen(seed, t.device)
    n = t.numel()
    for s in range(0, n, CHUNK):
        e = min(n, s + CHUNK)
        if t.dtype == torch.float32:
            t[s:e].normal_(0.0, std, generator=g)
        else:
            tmp = torch.empty(e - s, dtype=torch.float32, device=t.device)
            tmp.normal_(0.0, std, generator=g)
            t[s:e].copy_(tmp)
            del tmp
    return t


def fill_warm_moments_(m: torch.Tensor, v: torch.Tensor, grad_std: float, seed: int,
                       beta1: float = 0.9, beta2: float = 0.999, warm_steps: int = 100) -> None:
    """Draw first/second moments with the spread a warm start of ``warm_steps`` steps has.

    The moments are drawn directly, not computed by running the optimizer:
    after k steps of i.i.d. N(0, s^2) gradients the first moment is a zero-mean
    normal whose variance is s^2 (1-b1)^2 (1-b1^(2k)) / (1-b1^2), and the
    second moment is s^2 (1-b2) times a weighted sum of k chi-square(1)
    variables, drawn here as a Gamma variable with the same mean and variance.
    """
    var_m = grad_std ** 2 * (1 - beta1) ** 2 * (1 - beta1 ** (2 * warm_steps)) / (1 - beta1 ** 2)
    w = np.array([(1 - beta2) * beta2 ** j for j in range(warm_steps)])
    mean_v = grad_std ** 2 * w.sum()
    var_v = 2 * grad_std ** 4 * (w ** 2).sum()
    shape = mean_v ** 2 / var_v
    scale = var_v / mean_v
    fill_normal_(m, float(np.sqrt(var_m)), seed)
    g = _gen(seed + 1, v.device)
    n = v.numel()
    for s in range(0, n, CHUNK):
        e = min(n, s + CHUNK)
        conc = torch.full((e - s,), shape, dtype=torch.float32, device=v.device)
        # torch._standard_gamma takes no generator; derive it from a normal draw
        # stream instead: Gamma(k, theta) with k >= 1 via Marsaglia-Tsang.
        v[s:e].copy_(_gamma_mt(conc, g) * scale)
        del conc


def _gamma_mt(conc: torch.Tensor, g: torch.Generator) -> torch.Tensor:
    """Marsaglia & Tsang (2000) Gamma(k, 1) sampler for k >= 1, vectorised.

    Used only to draw synthetic second moments from a seeded generator.
    """
    d = conc - 1.0 / 3.0
    c = 1.0 / torch.sqrt(9.0 * d)
    out = torch.empty_like(conc)
    todo = torch.ones_like(conc, dtype=torch.bool)
    while bool(todo.any()):
        idx = todo.nonzero().squeeze(1)
        x = torch.empty(idx.numel(), dtype=conc.dtype, device=conc.device).normal_(generator=g)
        u = torch.empty(idx.numel(), dtype=conc.dtype, device=conc.device).uniform_(generator=g)
        vv = (1.0 + c[idx] * x) ** 3
        ok = (vv > 0) & (torch.log(u.clamp_min(1e-30)) <
                         0.5 * x * x + d[idx] - d[idx] * vv + d[idx] * torch.log(vv.clamp_min(1e-30)))
        take = idx[ok]
        out[take] = d[take] * vv[ok]
        todo[take] = False
    return out


# 16-bit encodings of the three non-finite values, per format.
NONFINITE_BITS = {
    torch.float16: (0x7C00, 0xFC00, 0x7E00),   # +inf, -inf, NaN
    torch.bfloat16: (0x7F80, 0xFF80, 0x7FC0),
}


def inject_nonfinite_(g16: torch.Tensor, prob: float, seed: int) -> np.ndarray:
    """Set each element independently with probability ``prob`` to +inf, -inf or NaN.

    Returns the sorted injected positions.  Draws are made on the host (numpy):
    a binomial count, then uniform positions and uniform choices of value.
    """
    rng = np.random.default_rng(seed)
    n = g16.numel()
    k = int(rng.binomial(n, prob))
    pos = np.unique(rng.integers(0, n, size=k, dtype=np.int64))
    which = rng.integers(0, 3, size=pos.size)
    bits = np.array(NONFINITE_BITS[g16.dtype], dtype=np.int64)[which]
    if pos.size:
        idx = torch.from_numpy(pos).to(g16.device)
        vals = torch.from_numpy(bits.astype(np.uint16).view(np.int16)).to(g16.device)
        g16.view(torch.int16).index_copy_(0, idx, vals)
    return pos


def spread_f32(n: int, seed: int, exp_lo: int, exp_hi: int, signed: bool = True) -> np.ndarray:
    """n FP32 values whose biased exponent fields are uniform in [exp_lo, exp_hi]
    (0 = zero and subnormals), with uniform significand bits and, if signed, a
    random sign: inputs that reach every binade of a chosen range, from the
    subnormals up.  A subnormal's significand is shifted right by a uniform 0
    to 22 bits, so the subnormals spread over all of their binades too."""
    rng = np.random.default_rng(seed)
    exp = rng.integers(exp_lo, exp_hi + 1, n, dtype=np.uint32)
    frac = rng.integers(0, 1 << 23, n, dtype=np.uint32)
    shift = rng.integers(0, 23, n, dtype=np.uint32)
    frac = np.where(exp == 0, frac >> shift, frac).astype(np.uint32)
    sign = rng.integers(0, 2, n, dtype=np.uint32) if signed else np.zeros(n, np.uint32)
    return ((sign << 31) | (exp << 23) | frac).view(np.float32)


def gpt2_small_shapes() -> list[tuple[str, tuple[int, ...]]]:
    """GPT-2 small's parameter tensors in flat order (148 tensors, 124,439,808 params).

    vocab 50257, context 1024, width 768, 12 blocks, MLP width 3072, tied head.
    """
    d, ff, vocab, ctx = 768, 3072, 50257, 1024
    shapes = [("wte", (vocab, d)), ("wpe", (ctx, d))]
    for i in range(12):
        h = f"h{i}"
        shapes += [
            (f"{h}.ln_1.w", (d,)), (f"{h}.ln_1.b", (d,)),
            (f"{h}.attn.c_attn.w", (d, 3 * d)), (f"{h}.attn.c_attn.b", (3 * d,)),
            (f"{h}.attn.c_proj.w", (d, d)), (f"{h}.attn.c_proj.b", (d,)),
            (f"{h}.ln_2.w", (d,)), (f"{h}.ln_2.b", (d,)),
            (f"{h}.mlp.c_fc.w", (d, ff)), (f"{h}.mlp.c_fc.b", (ff,)),
            (f"{h}.mlp.c_proj.w", (ff, d)), (f"{h}.mlp.c_proj.b", (d,)),
        ]
    shapes += [("ln_f.w", (d,)), ("ln_f.b", (d,))]
    return shapes


@dataclass(frozen=True)
class Workload:
    cfg: int
    name: str
    psi: int
    n: int
    ranks: tuple[int, ...]
    dtype: str                  # "f16" or "bf16"
    lr: float
    beta1: float
    beta2: float
    eps: float
    weight_decay: float
    loss_scale: float
    steps: int
    grad_std: float
    master_std: float = 0.02
    warm_steps: int = 0         # >0: moments drawn as if warm-started
    inject_prob: float = 0.0    # >0: non-finite injection on even 1-based steps
    extra: dict = field(default_factory=dict)

    @property
    def torch_dtype(self):
        return torch.float16 if self.dtype == "f16" else torch.bfloat16


WORKLOADS = {
    1: Workload(1, "flat1M_n8_rank3_f16_adam", 1_000_000, 8, (3,), "f16",
                1e-3, 0.9, 0.999, 1e-8, 0.0, 1.0, 3, 1e-3),
    2: Workload(2, "gpt2small_flat_n8_f16_adamw", 124_439_808, 8, tuple(range(8)), "f16",
                1e-3, 0.9, 0.999, 1e-8, 0.01, 1024.0, 10, 1e-3),
    3: Workload(3, "flat7.5B_n8_bf16_adamw_warm", 7_500_000_000, 8, (1,), "bf16",
                3e-4, 0.9, 0.999, 1e-8, 0.01, 1.0, 20, 1e-4, warm_steps=100),
    4: Workload(4, "flat10B_n1_f16_adamw", 10_000_000_000, 1, (0,), "f16",
                1e-4, 0.9, 0.999, 1e-8, 0.1, 65536.0, 5, 1e-3),
    5: Workload(5, "ragged8.81B_n64_rank63_f16_adam_overflow", 8_810_000_003, 64, (63,), "f16",
                1e-3, 0.9, 0.999, 1e-8, 0.0, 65536.0, 10, 1e-3, inject_prob=1e-7),
    # the pages' plain data-parallel example: 1.5e9 parameters, all 16 B/param
    # of state on one rank (24 GB)
    6: Workload(6, "flat1.5B_n1_bf16_adamw", 1_500_000_000, 1, (0,), "bf16",
                3e-4, 0.9, 0.999, 1e-8, 0.01, 1.0, 10, 1e-4),
}


def to_numpy_u16(t: torch.Tensor) -> np.ndarray:
    """Host copy of a 16-bit tensor as raw uint16 bit patterns."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16).copy()
