"""GPU parity where the step's quotients by per-call constants fall back to a
division.

The step forms g / S (S not a power of two), m / bc1 and v / bc2 as an FP64
reciprocal product rounded once to FP32, and divides only where that result is
below 2^-125 in magnitude with a non-zero numerator.  Realistic shards never
get there, so these cases put it there on purpose: BF16 and FP32 gradients
spread over the FP32 subnormal range, and moments that start subnormal or
tiny, mixed with ordinary values in the same vectors (so that lanes of one
wave take different paths).  Host-controlled calls with S a power of two and
not, the device-controlled sequence (S read on the device), the vector and the
element-wise kernels: the state after three steps must equal the oracle's bit
for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import zero_sharded_mixed_shard_amd as zs
from gpu_util import GuardedView, f32, log, u16

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TD = {"f16": torch.float16, "bf16": torch.bfloat16}
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
COUNT = 5003        # two 2048-element tiles, a ragged tail and a head
STEPS = 3
TINY = 2.0 ** -125


# Elements that get tiny values in every array (gradients, m, v), so that
# the moments stay tiny after an update; the others get ordinary values.
MASK = np.random.default_rng(777).random(COUNT) < 0.5


def mixed(tiny: np.ndarray, seed: int, std: float) -> np.ndarray:
    """Tiny values where MASK is set, N(0, std) draws elsewhere."""
    normal = (np.random.default_rng(seed).standard_normal(COUNT) * std).astype(np.float32)
    return np.where(MASK, tiny, normal).astype(np.float32)


def grads(kind: str, step: int) -> np.ndarray:
    """Host gradients: uint16 patterns (f16, bf16) or FP32 values (g32)."""
    seed = 500 + step
    if kind == "f16":       # FP16 has no values that small: zero there instead
        g = u16(synth.fill_normal_(torch.empty(COUNT, dtype=torch.float16), 1e-3, seed))
        return np.where(MASK, np.uint16(0), g).astype(np.uint16)
    tiny = synth.spread_f32(COUNT, seed, 0, 2)       # subnormals and the two lowest binades
    vals = mixed(tiny, seed + 50, 1e-3)
    if kind == "g32":
        return vals
    return (vals.view(np.uint32) >> 16).astype(np.uint16)   # BF16: the top half


def start_state():
    master = synth.fill_normal_(torch.empty(COUNT), 0.02, 41).numpy().copy()
    m = mixed(synth.spread_f32(COUNT, 42, 0, 2), 43, 1e-4)
    ordinary = np.square(np.random.default_rng(45).standard_normal(COUNT) * 1e-4)
    v = np.where(MASK, synth.spread_f32(COUNT, 44, 0, 2, signed=False), ordinary)
    return master, m, v.astype(np.float32)


def tiny_quotients(kind, S):
    """How many unscaled gradients and first-step moments land below 2^-125 (FP64)."""
    g = grads(kind, 1)
    gf = (g.astype(np.float64) if kind == "g32" else
          oracle.decode16(g, kind).astype(np.float64)) / S
    _, m, v = start_state()
    bc1 = 1.0 - HP["beta1"]
    bc2 = 1.0 - HP["beta2"]
    m1 = (HP["beta1"] * m.astype(np.float64) + (1 - HP["beta1"]) * gf) / bc1
    v1 = (HP["beta2"] * v.astype(np.float64) + (1 - HP["beta2"]) * gf * gf) / bc2

    def tiny(x):
        return int(np.count_nonzero((x != 0) & (np.abs(x) < TINY)))

    return tiny(gf), tiny(m1), tiny(v1)


def run(kind: str, wdt: str, S: float, control: str, phases: dict):
    g32 = kind == "g32"
    gt = torch.float32 if g32 else TD[kind]
    V = {"g": GuardedView(COUNT, gt, phases["g"], DEV)}
    for k in ("master", "m", "v"):
        V[k] = GuardedView(COUNT, torch.float32, phases[k], DEV)
    V["w16"] = GuardedView(COUNT, TD[wdt], phases["w16"], DEV)
    master, m, v = start_state()
    for k, a in (("master", master), ("m", m), ("v", v)):
        V[k].view.copy_(torch.from_numpy(a).to(DEV))
    V["w16"].view.zero_()
    ref = dict(master=master.copy(), m=m.copy(), v=v.copy(), w16=np.zeros(COUNT, np.uint16))
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    ctl = zs.device_ctl_new(S, DEV) if control == "device" else None
    bias = zs.zero_bias_corrections(HP["beta1"], HP["beta2"], 1, 8).to(DEV)
    for t in range(1, STEPS + 1):
        gh = grads(kind, t)
        if g32:
            V["g"].view.copy_(torch.from_numpy(gh).to(DEV))
        else:
            V["g"].view.copy_(torch.from_numpy(gh.view(np.int16)).view(TD[kind]).to(DEV))
        if control == "device":
            if g32:
                zs.zero_overflow_check_g32_dev(V["g"].view, COUNT, 1, 0, ctl)
            else:
                zs.zero_overflow_check_dev(V["g"].view, COUNT, 1, 0, ctl)
            zs.zero_scaler_update_dev(ctl, bias, 1)
            step = zs.zero_adam_step_g32_dev if g32 else zs.zero_adam_step_dev
            step(V["w16"].view, V["g"].view, V["master"].view, V["m"].view, V["v"].view,
                 COUNT, 1, 0, ctl=ctl, **HP)
        else:
            step = zs.zero_adam_step_g32 if g32 else zs.zero_adam_step
            step(V["w16"].view, V["g"].view, V["master"].view, V["m"].view, V["v"].view,
                 COUNT, 1, 0, step=t, loss_scale=S, found_inf=flag, **HP)
        if g32:
            oracle.adam_step_g32(ref["w16"], gh, ref["master"], ref["m"], ref["v"], wdt,
                                 step=t, loss_scale=S, **HP)
        else:
            oracle.adam_step(ref["w16"], gh, ref["master"], ref["m"], ref["v"], kind,
                             step=t, loss_scale=S, **HP)
    torch.cuda.synchronize()
    if control == "device":
        c = zs.device_ctl_read(ctl)
        assert (c.status, c.scaler.step, c.scaler.loss_scale) == (0, STEPS, S)
    got = dict(master=f32(V["master"].view), m=f32(V["m"].view), v=f32(V["v"].view),
               w16=u16(V["w16"].view))
    for k in ("master", "m", "v"):
        diff = np.count_nonzero(got[k].view(np.uint32) != ref[k].view(np.uint32))
        assert diff == 0, (k, kind, wdt, S, control, phases, diff)
    assert np.array_equal(got["w16"], ref["w16"]), ("w16", kind, wdt, S, control, phases)
    for k, gv in V.items():
        assert gv.guards_intact(), (k, kind, S, control, phases)


EQUAL = dict.fromkeys(("g", "master", "m", "v", "w16"), 3)
MIXED = {"g": 1, "master": 0, "m": 2, "v": 3, "w16": 1}


@pytest.mark.parametrize("control", ["host", "device"])
@pytest.mark.parametrize("S", [3.0, 1000.0, 1.0, 2.0 ** -20])
@pytest.mark.parametrize("kind,wdt", [("bf16", "bf16"), ("f16", "f16"), ("g32", "f16"),
                                      ("g32", "bf16")])
def test_fallback_divisions_match_the_oracle(kind, wdt, S, control):
    log(f"quotient fallback kind={kind} weights={wdt} S={S} control={control}")
    n_g, n_m, n_v = tiny_quotients(kind, S)
    # bias-corrected moments below 2^-125 after the first update (m only while
    # the unscaled gradients stay small), and unscaled gradients below 2^-125
    assert n_v > 100, n_v
    assert n_m > 100 or (kind != "f16" and S < 1.0), n_m
    assert n_g > 100 or kind == "f16" or S < 1.0, n_g
    run(kind, wdt, S, control, EQUAL)


@pytest.mark.parametrize("S", [3.0, 1.0])
@pytest.mark.parametrize("kind,wdt", [("bf16", "bf16"), ("g32", "f16")])
def test_fallback_divisions_in_the_element_wise_kernel(kind, wdt, S):
    log(f"quotient fallback, element-wise kernel kind={kind} S={S}")
    for control in ("host", "device"):
        run(kind, wdt, S, control, MIXED)
