"""Pins for the parity bar's ulp distance (the tolerance every GPU test applies)."""
import numpy as np

import oracle


def test_ulp_distance32_counts_representable_steps():
    x = np.float32(1.0)
    up = [x]
    for _ in range(5):
        up.append(np.nextafter(up[-1], np.float32(2)))
    d = oracle.ulp_distance32(np.array(up[:1] * 6, np.float32), np.array(up, np.float32))
    assert list(d) == [0, 1, 2, 3, 4, 5]


def test_ulp_distance32_across_zero_and_nan():
    tiny = np.float32(1.4e-45)  # smallest subnormal
    a = np.array([0.0, -0.0, tiny, -tiny, np.nan, np.nan, 1.0], np.float32)
    b = np.array([-0.0, 0.0, -tiny, tiny, np.nan, 1.0, np.nan], np.float32)
    d = oracle.ulp_distance32(a, b)
    assert list(d[:5]) == [0, 0, 2, 2, 0]
    assert d[5] > 2 ** 30 and d[6] > 2 ** 30


def test_ulp_distance16_f16_and_bf16():
    a = np.array([0x3C00, 0x3C00, 0x8000, 0x0001, 0x7E00], np.uint16)
    b = np.array([0x3C01, 0x3BFF, 0x0000, 0x8001, 0x7E01], np.uint16)
    assert list(oracle.ulp_distance16(a, b, "f16")) == [1, 1, 0, 2, 0]
    a = np.array([0x3F80, 0x7FC0], np.uint16)
    b = np.array([0x3F82, 0x3F80], np.uint16)
    d = oracle.ulp_distance16(a, b, "bf16")
    assert d[0] == 2 and d[1] > 2 ** 30
