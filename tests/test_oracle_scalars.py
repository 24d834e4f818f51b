"""Pins of the oracle's per-call scalars against exact rational arithmetic.

The bias corrections 1 - beta^t are formed in FP64 and rounded once to FP32
(reading R-6 of "Training models too big for one GPU: ZeRO & FSDP", "Adam, and
why it's expensive": the bias-corrected moments divide by 1 - beta^t).  Here
the exact value of 1 - beta^t (beta taken as the FP32 number it is) is
computed with Python fractions and rounded to FP32 by hand (to nearest, ties
to even); the oracle must give exactly that, except where the exact value lies
so close to an FP32 rounding midpoint that an FP64 evaluation cannot decide it
(none occur in these grids).  The same check tells the reading apart from the
plausible slip of evaluating the power in FP32.  1 - beta and 1 - lr*wd are
FP32 operations; they are checked against their exact values too.
"""
from fractions import Fraction

import numpy as np

import oracle

F32 = np.float32


def round_f32(x: Fraction) -> np.float32:
    """x rounded to the nearest FP32 number, ties to even (normal range)."""
    q = F32(float(x))                     # within one FP32 ulp of the answer
    cands = {q, np.nextafter(q, F32(np.inf)), np.nextafter(q, F32(-np.inf))}
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - x),
                                     int(np.array(c, F32).view(np.uint32)) & 1))
    return F32(best)


def midpoint_distance(x: Fraction) -> Fraction:
    """Relative distance from x to the nearest FP32 rounding midpoint."""
    q = round_f32(x)
    lo, hi = np.nextafter(q, F32(-np.inf)), np.nextafter(q, F32(np.inf))
    mids = [(Fraction(float(q)) + Fraction(float(lo))) / 2,
            (Fraction(float(q)) + Fraction(float(hi))) / 2]
    return min(abs(x - m) for m in mids) / abs(x)


BETAS = [0.9, 0.95, 0.98, 0.99, 0.995, 0.999, 0.9995, 0.9999, 0.5, 0.25, 0.0]


def grid():
    rng = np.random.default_rng(62)
    betas = [F32(b) for b in BETAS] + [F32(x) for x in rng.random(12)]
    ts = list(range(1, 80)) + [100, 101, 120, 257, 500, 1000, 2000]
    return betas, ts


def test_bias_corrections_are_the_exact_value_rounded_once():
    betas, ts = grid()
    undecidable = 0
    fp32_pow_differs = 0
    for b in betas:
        fb = Fraction(float(b))
        p = Fraction(1)
        prev = 0
        for t in ts:
            p *= fb ** (t - prev)
            prev = t
            exact = 1 - p
            if exact == 0:
                continue
            # a value FP64 holds exactly (0.5^t, say) is decided exactly, ties to even;
            # otherwise it must lie clear of every FP32 midpoint
            if Fraction(float(exact)) != exact and midpoint_distance(exact) < Fraction(1, 2 ** 50):
                undecidable += 1
                continue
            want = round_f32(exact)
            got = oracle.step_scalars(1e-3, float(b), float(b), 0.0, t)
            assert F32(got.bc1) == want and F32(got.bc2) == want, (float(b), t, got, want)
            if F32(1) - F32(b) ** t != want:
                fp32_pow_differs += 1
    assert undecidable == 0
    # the pin separates the reading from an FP32 evaluation of the power
    assert fp32_pow_differs > 50, fp32_pow_differs


def test_one_minus_beta_and_the_decay_are_fp32_operations():
    rng = np.random.default_rng(63)
    for b in [F32(x) for x in BETAS] + [F32(x) for x in rng.random(50)]:
        s = oracle.step_scalars(1e-3, float(b), float(b), 0.0, 1)
        assert F32(s.omb1) == round_f32(1 - Fraction(float(b))) == F32(s.omb2)
    for lr, wd in [(1e-3, 0.01), (1e-4, 0.1), (3e-4, 0.01), (-1e-3, 0.1), (1e-2, 0.5),
                   (0.37, 0.11)] + [(float(x), float(y)) for x, y in rng.random((30, 2))]:
        s = oracle.step_scalars(lr, 0.9, 0.999, wd, 1)
        lw = round_f32(Fraction(float(F32(lr))) * Fraction(float(F32(wd))))
        assert F32(s.decay) == round_f32(1 - Fraction(float(lw))), (lr, wd)
