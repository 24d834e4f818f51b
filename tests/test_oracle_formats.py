"""Pins for the oracle's 16-bit conversions.

The oracle converts from the IEEE field definitions.  Pins: numpy's float16
(IEEE binary16, round to nearest even) and torch's CPU bfloat16 (round to
nearest even) on every 16-bit pattern, on every rounding case class of FP32
inputs and on all 2^32 FP32 patterns, plus the format table the first page prints
(tests/golden/formats.tsv) and its lost-update example
(tests/golden/lost_update.tsv).
"""
import os

import numpy as np
import pytest
import torch

import oracle

ALL16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def _same_bits_or_both_nan(a_f32, b_f32):
    a_nan, b_nan = np.isnan(a_f32), np.isnan(b_f32)
    assert np.array_equal(a_nan, b_nan)
    ok = ~a_nan
    assert np.array_equal(a_f32[ok].view(np.uint32), b_f32[ok].view(np.uint32))


def test_decode_f16_all_patterns():
    ref = ALL16.view(np.float16).astype(np.float32)
    _same_bits_or_both_nan(oracle.decode16(ALL16, "f16"), ref)


def test_decode_bf16_all_patterns():
    ref = torch.from_numpy(ALL16.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    _same_bits_or_both_nan(oracle.decode16(ALL16, "bf16"), ref)
    # bf16 is the top half of a binary32 pattern
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok].view(np.uint32), (ALL16.astype(np.uint32) << 16)[ok])


def _rounding_cases(round_bits_for_exponent, rng):
    """FP32 patterns covering each rounding case at the rounding position.

    For every sign and every biased FP32 exponent, the bits below the rounding
    position take the values 0, 1, half-1, half, half+1 and all-ones, with
    both parities of the kept lsb and random kept bits above.
    """
    out = []
    for sign in (0, 1):
        for e in range(0, 256):
            k = round_bits_for_exponent(e)  # number of discarded low bits (<= 24)
            if k <= 0:
                continue
            half = 1 << (k - 1)
            lows = {0, 1, half - 1, half, half + 1, (1 << k) - 1}
            if k >= 24:
                lows = {x & ((1 << 23) - 1) for x in lows}
            kept_bits = max(0, 23 - k - 1)
            highs = rng.integers(0, 1 << kept_bits, size=24) if kept_bits else np.zeros(1, int)
            for hi in highs:
                for lsb in (0, 1):
                    for lo in lows:
                        mant = ((int(hi) << (k + 1)) | (lsb << k) | lo) & ((1 << 23) - 1)
                        out.append((sign << 31) | (e << 23) | mant)
    return np.array(out, dtype=np.uint32)


def _f16_round_bits(e):
    # FP32 biased exponent e -> unbiased E = e - 127; binary16 keeps 10 fraction
    # bits for E >= -14 and fewer in its subnormal range.
    E = e - 127
    if E >= -14:
        return 13
    return min(24, 13 + (-14 - E))


def _bf16_round_bits(e):
    return 16  # same exponent range as FP32: rounding always at bit 16


def test_encode_f16_rounding_cases_and_random():
    rng = np.random.default_rng(7)
    cases = _rounding_cases(_f16_round_bits, rng)
    rand = rng.integers(0, 1 << 32, size=1 << 21, dtype=np.uint64).astype(np.uint32)
    x = np.concatenate([cases, rand]).view(np.float32)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    got = oracle.encode16(x, "f16")
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    # NaN stays NaN (quiet, sign kept)
    assert np.all((got[nan] & 0x7C00) == 0x7C00) and np.all(got[nan] & 0x0200)
    assert np.array_equal(got[nan] >> 15, x[nan].view(np.uint32) >> 31)


def test_encode_bf16_rounding_cases_and_random():
    rng = np.random.default_rng(8)
    cases = _rounding_cases(_bf16_round_bits, rng)
    rand = rng.integers(0, 1 << 32, size=1 << 21, dtype=np.uint64).astype(np.uint32)
    x = np.concatenate([cases, rand]).view(np.float32)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.encode16(x, "bf16")
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7F80) == 0x7F80) and np.all(got[nan] & 0x0040)


def _every_fp32_pattern(fmt, reference):
    """oracle.encode16 against a reference on all 2^32 FP32 bit patterns.

    Non-NaN inputs must give the reference's bits; NaN inputs a quiet NaN of
    the same sign.  Chunks run on a thread pool (the conversions release the
    interpreter lock)."""
    from concurrent.futures import ThreadPoolExecutor

    chunk = 1 << 20
    exp_field, quiet = (0x7C00, 0x0200) if fmt == "f16" else (0x7F80, 0x0040)
    offsets = np.arange(chunk, dtype=np.uint32)

    def run(c):
        bits = offsets + np.uint32(c * chunk)
        x = bits.view(np.float32)
        got = oracle.encode16(x, fmt)
        want = reference(x)
        nan = np.isnan(x)
        bad = np.count_nonzero(got[~nan] != want[~nan])
        bad += np.count_nonzero(((got[nan] & exp_field) != exp_field) | ((got[nan] & quiet) == 0) |
                                ((got[nan] >> 15) != (bits[nan] >> 31)))
        return bad

    workers = min(8, os.cpu_count() or 1)
    with ThreadPoolExecutor(workers) as pool:
        bad = sum(pool.map(run, range((1 << 32) // chunk)))
    assert bad == 0


def test_encode_f16_every_fp32_pattern():
    def ref(x):
        with np.errstate(over="ignore"):
            return x.astype(np.float16).view(np.uint16)
    _every_fp32_pattern("f16", ref)


def test_encode_bf16_every_fp32_pattern():
    def ref(x):
        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    _every_fp32_pattern("bf16", ref)


def test_subnormal_f16_survives():
    # a typical gradient of 1e-6 is an FP16 subnormal; it must round, not flush
    x = np.array([1e-6, -3e-7, 6e-8, 2.9e-8, 3.0e-8], np.float32)
    got = oracle.encode16(x, "f16")
    assert np.array_equal(got, x.astype(np.float16).view(np.uint16))
    assert got[0] != 0 and got[2] == 1


def _golden_rows(golden_dir, name):
    rows = []
    with open(os.path.join(golden_dir, name)) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            rows.append(line.rstrip("\n").split("\t"))
    return rows


def _pow2(s):
    assert s.startswith("2^")
    return 2.0 ** int(s[2:])


def test_format_table(golden_dir):
    rows = {r[0]: r for r in _golden_rows(golden_dir, "formats.tsv")}
    # FP16: 1/5/10 bits, largest finite 65,504, gap after 1.0 = 2^-10
    _, s, e, m, big, gap = rows["fp16"]
    one = oracle.encode16(np.array([1.0], np.float32), "f16")[0]
    assert one == (15 << 10)  # exponent field = bias, fraction 0
    nxt = oracle.decode16(np.array([one + 1], np.uint16), "f16")[0]
    assert nxt - 1.0 == _pow2(gap) == 2.0 ** -int(m)
    largest = oracle.decode16(np.array([((1 << int(e)) - 2) << int(m) | ((1 << int(m)) - 1)],
                                       np.uint16), "f16")[0]
    assert largest == float(big)
    assert oracle.encode16(np.array([65519.99], np.float32), "f16")[0] == 0x7BFF
    assert oracle.encode16(np.array([65520.0], np.float32), "f16")[0] == 0x7C00  # overflow to inf
    # BF16: 1/8/7 bits, largest finite ~3.4e38, gap after 1.0 = 2^-7
    _, s, e, m, big, gap = rows["bf16"]
    one = oracle.encode16(np.array([1.0], np.float32), "bf16")[0]
    nxt = oracle.decode16(np.array([one + 1], np.uint16), "bf16")[0]
    assert nxt - 1.0 == _pow2(gap) == 2.0 ** -int(m)
    largest = oracle.decode16(np.array([0x7F7F], np.uint16), "bf16")[0]
    assert f"{largest:.1e}" == "3.4e+38" and float(big) == 3.4e38
    # FP32 gap after one, for completeness of the table
    _, s, e, m, big, gap = rows["fp32"]
    assert float(np.nextafter(np.float32(1), np.float32(2))) - 1.0 == _pow2(gap)


def test_lost_update(golden_dir):
    (w, upd, gap, result), = _golden_rows(golden_dir, "lost_update.tsv")
    x = np.array([np.float32(w) + np.float32(upd)], np.float32)
    bits = oracle.encode16(x, "f16")
    assert oracle.decode16(bits, "f16")[0] == float(result)
    one = oracle.encode16(np.array([1.0], np.float32), "f16")[0]
    g = oracle.decode16(np.array([one + 1], np.uint16), "f16")[0] - 1.0
    assert round(g, 5) == float(gap)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_roundtrip_16_to_32_to_16(dtype):
    f = oracle.decode16(ALL16, dtype)
    back = oracle.encode16(f, dtype)
    nan = np.isnan(f)
    assert np.array_equal(back[~nan], ALL16[~nan])
