"""Pins for the oracle's shard layout and per-stage byte accounting.

Pins: brute-force enumeration of "chunk i of an equally chunked flat buffer
belongs to rank i" on tiny inputs; the stage closed forms 16psi, 4psi+12psi/N,
2psi+14psi/N, 16psi/N whenever N divides psi; and every memory figure the pages
print (tests/golden/memory_accounting.tsv).
"""
import os
from fractions import Fraction

import pytest

import oracle


def brute_force_layout(psi, n):
    """Enumerate every flat index and hand it to its chunk; no division used.

    The chunk size is the smallest S whose n chunks hold all psi elements
    (searched upward), and index j lands in chunk k when k*S <= j < (k+1)*S.
    """
    S = 1
    while n * S < psi:
        S += 1
    owned = [[] for _ in range(n)]
    k, start = 0, 0
    for j in range(psi):
        while j >= start + S:
            k += 1
            start += S
        owned[k].append(j)
    return S, owned


@pytest.mark.parametrize("psi", list(range(1, 80)) + [97, 128, 255, 256])
def test_layout_matches_brute_force(psi):
    for n in range(1, 33):
        S, owned = brute_force_layout(psi, n)
        seen = []
        total_pad = 0
        for r in range(n):
            lay = oracle.layout(psi, n, r)
            assert lay.shard == S
            assert lay.offset == r * S
            assert lay.count == len(owned[r])
            if owned[r]:
                assert owned[r][0] == lay.offset
                assert owned[r] == list(range(lay.offset, lay.offset + lay.count))
            assert lay.count <= S
            assert lay.pad == S - lay.count
            assert lay.padded_total == n * S
            total_pad += lay.pad
            seen.extend(range(lay.offset, lay.offset + lay.count))
        # disjoint and covering [0, psi)
        assert seen == list(range(psi))
        assert total_pad == n * S - psi
        assert total_pad < n


def test_empty_trailing_ranks():
    # psi = 10 over 8 ranks: chunks of 2, ranks 5..7 own nothing.
    counts = [oracle.layout(10, 8, r).count for r in range(8)]
    assert counts == [2, 2, 2, 2, 2, 0, 0, 0]


@pytest.mark.parametrize("psi,n", [(1_000_000, 8), (124_439_808, 8), (7_500_000_000, 8),
                                   (10_000_000_000, 1), (7_500_000_000, 64),
                                   (10_000_000_000, 64), (3 * 2**40, 96), (12, 12), (4096, 1)])
def test_stage_bytes_closed_forms_when_n_divides_psi(psi, n):
    assert psi % n == 0
    for r in (0, n - 1):
        lay = oracle.layout(psi, n, r)
        P, N = Fraction(psi), Fraction(n)
        assert lay.bytes_dp == 16 * P
        assert lay.bytes_z1 == 4 * P + 12 * P / N
        assert lay.bytes_z2 == 2 * P + 14 * P / N
        assert lay.bytes_z3 == 16 * P / N
        # per-parameter forms of the stage-3 page: 16, 4+12/N, 2+14/N, 16/N
        assert Fraction(lay.bytes_z1) / P == 4 + Fraction(12) / N
        assert Fraction(lay.bytes_z2) / P == 2 + Fraction(14) / N
        assert Fraction(lay.bytes_z3) / P == Fraction(16) / N


@pytest.mark.parametrize("psi,n", [(8_810_000_003, 64), (10, 8), (1_000_003, 8), (2**33 + 1, 7)])
def test_stage_bytes_with_padding_exceed_closed_forms_by_little(psi, n):
    lay = oracle.layout(psi, n, 0)
    P, N = Fraction(psi), Fraction(n)
    assert lay.bytes_dp == 16 * P
    assert 0 <= lay.bytes_z1 - (4 * P + 12 * P / N) < 4 * n + 12
    assert 0 <= lay.bytes_z2 - (2 * P + 14 * P / N) < 2 * n + 14
    assert 0 <= lay.bytes_z3 - 16 * P / N < 16


def _read_golden(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "memory_accounting.tsv")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            psi, n, q, printed, tol, src = line.rstrip("\n").split("\t")
            rows.append((int(psi), int(n), q, printed, float(tol), src))
    return rows


def test_printed_memory_figures(golden_dir):
    rows = _read_golden(golden_dir)
    assert len(rows) >= 15
    for psi, n, q, printed, tol, src in rows:
        lay = oracle.layout(psi, n, 0)
        S = lay.shard
        value = {
            "dp": lay.bytes_dp,
            "z1": lay.bytes_z1,
            "z2": lay.bytes_z2,
            "z3": lay.bytes_z3,
            "floor_z1": lay.bytes_z1 - 12 * S,
            "floor_z2": lay.bytes_z2 - 14 * S,
            "grad16": 2 * psi,
        }[q] / 1e9
        decimals = len(printed.split(".")[1]) if "." in printed else 0
        if tol == 0:
            assert round(value, decimals) == float(printed), (q, psi, n, value, src)
        else:
            assert abs(value - float(printed)) <= tol, (q, psi, n, value, src)


def test_ragged_64bit_layout():
    lay = oracle.layout(8_810_000_003, 64, 63)
    assert (lay.shard, lay.offset, lay.count, lay.pad) == (137_656_251, 8_672_343_813,
                                                           137_656_190, 61)
    assert lay.offset % 8 == 5
    assert lay.padded_total == 8_810_000_064
    big = oracle.layout(10_000_000_000, 1, 0)
    assert (big.shard, big.offset, big.count, big.pad) == (10**10, 0, 10**10, 0)
    assert big.bytes_dp == 160 * 10**9


@pytest.mark.parametrize("args", [(0, 8, 0), (10, 0, 0), (10, 8, 8), (2**56 + 1, 8, 0)])
def test_invalid_layout_arguments(args):
    with pytest.raises(ValueError):
        oracle.layout(*args)
