"""Property-based checks (hypothesis) of the shard layout, the accounting and
the re-shard plan over their whole argument domain: psi up to 2^56, N up to
2^32 - 1, any rank.

The layout properties characterise the partition the pages describe (the
flat buffer cut into N equal chunks, chunk i owned by rank i, the padding at
the tail) without restating its formula: the chunks tile [0, N*S) in rank
order; S is the smallest chunk size whose N chunks cover psi; every element
has exactly one owner; at most one rank is ragged and every rank after it is
empty; and the per-rank bytes order as the stages shard more (plain data
parallelism >= stage 1 >= stage 2 >= stage 3).  The library's layout,
accounting and re-shard plan must agree with the oracle and with these
properties for every drawn argument.
"""
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
import zero_sharded_mixed_shard_amd as zs

MAX_PSI = 1 << 56
SETTINGS = settings(max_examples=400, deadline=None,
                    suppress_health_check=[HealthCheck.too_slow])

psi_st = st.one_of(st.integers(1, 2000), st.integers(1, MAX_PSI))
n_st = st.one_of(st.integers(1, 70), st.integers(1, 2 ** 32 - 1))


@st.composite
def layout_args(draw):
    psi, n = draw(psi_st), draw(n_st)
    S = -(-psi // n)
    ragged = min(n - 1, (psi - 1) // S)              # the last rank that owns anything
    rank = draw(st.one_of(st.integers(0, n - 1),
                          st.sampled_from(sorted({0, n - 1, ragged, min(n - 1, ragged + 1)}))))
    return psi, n, rank


def _fields(lay):
    return (lay.psi, lay.shard, lay.offset, lay.count, lay.pad, lay.padded_total, lay.n,
            lay.rank, lay.bytes_dp, lay.bytes_z1, lay.bytes_z2, lay.bytes_z3)


@SETTINGS
@given(layout_args())
def test_layout_is_the_pages_partition(args):
    psi, n, r = args
    lay = oracle.layout(psi, n, r)
    S = lay.shard
    # n equal chunks of the smallest size that covers psi
    assert n * S >= psi and n * (S - 1) < psi and lay.padded_total == n * S
    # the chunks tile the padded buffer in rank order
    if r == 0:
        assert lay.offset == 0
    else:
        prev = oracle.layout(psi, n, r - 1)
        assert lay.offset == prev.offset + prev.shard and prev.shard == S
    if r == n - 1:
        assert lay.offset + S == lay.padded_total
    # the chunk's real part, then its padding
    assert 0 <= lay.count <= S and lay.count + lay.pad == S
    if lay.offset + S <= psi:
        assert lay.count == S                       # a chunk inside the buffer is full
    elif lay.offset >= psi:
        assert lay.count == 0                       # past the end: an empty rank
    else:
        assert lay.offset + lay.count == psi        # the ragged rank ends the buffer
    # stage bytes shrink as more is sharded
    assert lay.bytes_dp == 16 * psi
    assert 16 * lay.padded_total >= lay.bytes_z1 >= lay.bytes_z2 >= lay.bytes_z3 == 16 * S


@SETTINGS
@given(layout_args(), st.integers(0, MAX_PSI))
def test_every_element_has_exactly_one_owner(args, i):
    psi, n, _ = args
    i %= psi
    S = oracle.layout(psi, n, 0).shard
    owner = i // S
    lay = oracle.layout(psi, n, owner)
    assert lay.offset <= i < lay.offset + lay.count
    for k in (owner - 1, owner + 1):
        if 0 <= k < n:
            other = oracle.layout(psi, n, k)
            assert not (other.offset <= i < other.offset + other.count)


@SETTINGS
@given(layout_args())
def test_padding_only_at_the_tail(args):
    psi, n, r = args
    lay = oracle.layout(psi, n, r)
    if lay.count < lay.shard and r + 1 < n:
        assert oracle.layout(psi, n, r + 1).count == 0
    if r > 0:
        assert oracle.layout(psi, n, r - 1).count == lay.shard or lay.count == 0


@SETTINGS
@given(layout_args())
def test_library_layout_equals_oracle(args):
    assert _fields(zs.zero_shard_layout(*args)) == _fields(oracle.layout(*args))


@SETTINGS
@given(psi_st, st.integers(1, 1024), st.integers(0, 3), st.sampled_from([1, 2, 4, 8]))
def test_library_comm_volume_equals_oracle(psi, n, stage, eb):
    lib = zs.zero_comm_volume(psi, n, stage, eb)
    ref = oracle.comm_volume(psi, n, stage, eb)
    assert {k: lib[k] for k in ref} == ref


@SETTINGS
@given(st.integers(1, 2 ** 40), st.integers(1, 1024), st.integers(0, 2 ** 40),
       st.integers(0, 64), st.integers(0, 2 ** 40))
def test_library_peak_memory_equals_oracle(psi, n, unit, units, act):
    unit %= psi + 1
    assert zs.zero_peak_memory(psi, n, unit, units, act) == \
        oracle.peak_memory(psi, n, unit, units, act)


@SETTINGS
@given(st.one_of(st.integers(1, 5000), st.integers(1, 2 ** 48)), st.integers(1, 64),
       st.integers(1, 64), st.data())
def test_reshard_plan_reads_exactly_the_new_range(psi, n_old, n_new, data):
    r = data.draw(st.integers(0, n_new - 1))
    new = oracle.layout(psi, n_new, r)
    pieces = zs.zero_reshard_plan(psi, n_old, n_new, r)
    dst = 0
    last_src = -1
    for src_rank, src_first, dst_first, count in pieces:
        old = oracle.layout(psi, n_old, src_rank)
        assert count > 0 and dst_first == dst and src_rank > last_src
        assert src_first + count <= old.count                    # inside the old shard
        assert old.offset + src_first == new.offset + dst_first  # the same flat elements
        dst += count
        last_src = src_rank
    assert dst == new.count
