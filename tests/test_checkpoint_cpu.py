"""Sharded checkpoints (host side): round trip, integrity checks, the re-shard
plan against brute force, resharded reads, and resume invariance with the
oracle (N shards -> save -> N' shards -> continue equals the unsharded run).
"""
import os
import struct

import numpy as np
import pytest

import oracle
import zero_sharded_mixed_shard_amd as zs

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def state(count, seed):
    rng = np.random.default_rng(seed)
    return (rng.integers(0, 1 << 16, count, dtype=np.uint32).astype(np.uint16),
            rng.standard_normal(count).astype(np.float32),
            rng.standard_normal(count).astype(np.float32),
            rng.random(count).astype(np.float32))


def test_round_trip_and_info(tmp_path):
    psi, n = 1_000_003, 8
    for rank in (0, 7):
        cnt = oracle.layout(psi, n, rank).count
        st = state(cnt, rank)
        sc = zs.Scaler(2048.0, growth_interval=77, step=1234)
        sc.clean_steps = 5
        p = str(tmp_path / f"r{rank}.zshard")
        zs.zero_ckpt_write(p, psi, n, rank, "bf16", sc, *st)
        info = zs.zero_ckpt_read_info(p)
        assert (info.psi, info.n, info.rank, info.count, info.dtype) == (psi, n, rank, cnt, 1)
        assert info.offset == oracle.layout(psi, n, rank).offset
        assert (info.scaler.loss_scale, info.scaler.growth_interval, info.scaler.step,
                info.scaler.clean_steps) == (2048.0, 77, 1234, 5)
        zs.zero_ckpt_verify(p)
        back = zs.zero_ckpt_read(p, 0, cnt)
        for a, b in zip(st, back):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
        part = zs.zero_ckpt_read(p, 12345, 1000)
        for a, b in zip(st, part):
            assert np.array_equal(a[12345:13345].view(np.uint8), b.view(np.uint8))
        assert os.path.getsize(p) == 128 + 14 * cnt


def test_empty_rank_round_trip(tmp_path):
    p = str(tmp_path / "e.zshard")
    empty = [np.zeros(0, np.uint16)] + [np.zeros(0, np.float32)] * 3
    zs.zero_ckpt_write(p, 10, 8, 7, "f16", zs.Scaler(1.0), *empty)
    assert zs.zero_ckpt_read_info(p).count == 0
    zs.zero_ckpt_verify(p)


def test_overwrite_replaces_whole_file_and_failed_write_keeps_old(tmp_path):
    psi, n, rank = 50_000, 4, 2
    cnt = oracle.layout(psi, n, rank).count
    p = str(tmp_path / "w.zshard")
    first, second = state(cnt, 10), state(cnt, 11)
    zs.zero_ckpt_write(p, psi, n, rank, "f16", zs.Scaler(1.0, step=1), *first)
    zs.zero_ckpt_write(p, psi, n, rank, "f16", zs.Scaler(1.0, step=2), *second)
    assert sorted(os.listdir(tmp_path)) == ["w.zshard"]        # no temporary left behind
    assert zs.zero_ckpt_read_info(p).scaler.step == 2
    for a, b in zip(second, zs.zero_ckpt_read(p, 0, cnt)):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    # a write that cannot create its temporary file fails and leaves the old file whole
    os.mkdir(p + ".tmp")
    with pytest.raises(zs.ZeroError) as e:
        zs.zero_ckpt_write(p, psi, n, rank, "f16", zs.Scaler(1.0, step=3), *first)
    assert e.value.code == -5
    os.rmdir(p + ".tmp")
    zs.zero_ckpt_verify(p)
    assert zs.zero_ckpt_read_info(p).scaler.step == 2


def payload_hash(payload: bytes) -> int:
    """The file's payload hash from its definition: FNV-1a over 8-byte little-endian
    words in four lanes (word i to lane i mod 4), the lanes then folded in order."""
    mask, prime, start = (1 << 64) - 1, 0x100000001B3, 0xCBF29CE484222325
    padded = payload + b"\0" * (-len(payload) % 8)
    words = np.frombuffer(padded, dtype="<u8")
    lanes = [start] * 4
    for i, w in enumerate(words.tolist()):
        lanes[i % 4] = ((lanes[i % 4] ^ w) * prime) & mask
    h = start
    for x in lanes:
        h = ((h ^ x) * prime) & mask
    return h


@pytest.mark.parametrize("psi,n,rank", [(1_000, 4, 1), (1_003, 4, 3), (9, 8, 3), (10, 8, 6)])
def test_file_format_and_hash_follow_their_definition(tmp_path, psi, n, rank):
    # counts 250, 250, 2 and 0 elements: payloads of 3500, 3500, 28 and 0 bytes
    lay = oracle.layout(psi, n, rank)
    st = state(lay.count, psi + rank)
    p = str(tmp_path / "f.zshard")
    zs.zero_ckpt_write(p, psi, n, rank, "bf16", zs.Scaler(512.0, growth_interval=9, step=4), *st)
    raw = open(p, "rb").read()
    hdr, payload = raw[:128], raw[128:]
    assert hdr[:8] == b"ZSHARD01"
    version, dtype, psi_, n_, rank_, off, cnt, step, clean = struct.unpack_from("<IIQIIQQQQ", hdr, 8)
    scale, growth, nbytes, h = struct.unpack_from("<fIQQ", hdr, 64)
    assert (version, dtype, psi_, n_, rank_, off, cnt, step, clean) == \
        (2, 1, psi, n, rank, lay.offset, lay.count, 4, 0)
    assert (scale, growth, nbytes) == (512.0, 9, 14 * lay.count) and hdr[88:] == bytes(40)
    assert payload == b"".join(a.tobytes() for a in st)
    assert h == payload_hash(payload)


def test_integrity_errors(tmp_path):
    psi, n, rank = 10_000, 4, 1
    cnt = oracle.layout(psi, n, rank).count
    p = str(tmp_path / "x.zshard")
    zs.zero_ckpt_write(p, psi, n, rank, "f16", zs.Scaler(1.0), *state(cnt, 3))
    raw = open(p, "rb").read()
    # a flipped payload byte: the header still reads, the hash does not match
    bad = bytearray(raw)
    bad[128 + 5000] ^= 0x40
    q = str(tmp_path / "flip.zshard")
    open(q, "wb").write(bytes(bad))
    zs.zero_ckpt_read_info(q)
    with pytest.raises(zs.ZeroError) as e:
        zs.zero_ckpt_verify(q)
    assert e.value.code == -6
    # truncated, wrong magic, inconsistent layout fields
    for name, data in (("trunc", raw[:-4]), ("magic", b"X" + raw[1:]),
                       ("count", raw[:40] + (cnt + 1).to_bytes(8, "little") + raw[48:])):
        q = str(tmp_path / f"{name}.zshard")
        open(q, "wb").write(data)
        with pytest.raises(zs.ZeroError) as e:
            zs.zero_ckpt_read_info(q)
        assert e.value.code == -6, name
    with pytest.raises(zs.ZeroError) as e:
        zs.zero_ckpt_read_info(str(tmp_path / "missing.zshard"))
    assert e.value.code == -5
    with pytest.raises(zs.ZeroError) as e:
        zs.zero_ckpt_read(p, cnt - 10, 11)
    assert e.value.code == -1


def brute_plan(psi, n_old, n_new, r_new):
    """Walk the new rank's flat indices; group runs that come from one old shard."""
    S = oracle.layout(psi, n_old, 0).shard
    lay = oracle.layout(psi, n_new, r_new)
    pieces = []
    for j in range(lay.offset, lay.offset + lay.count):
        k, pos, dst = j // S, j % S, j - lay.offset
        if pieces and pieces[-1][0] == k and pieces[-1][1] + pieces[-1][3] == pos:
            pieces[-1] = (k, pieces[-1][1], pieces[-1][2], pieces[-1][3] + 1)
        else:
            pieces.append((k, pos, dst, 1))
    return pieces


def test_reshard_plan_brute_force():
    for psi in list(range(1, 40)) + [97, 1000]:
        for n_old in range(1, 10):
            for n_new in range(1, 10):
                for r in range(n_new):
                    assert zs.zero_reshard_plan(psi, n_old, n_new, r) == \
                        brute_plan(psi, n_old, n_new, r), (psi, n_old, n_new, r)


@pytest.mark.parametrize("psi,n_old,n_new", [(100_003, 8, 5), (100_003, 1, 8), (100_003, 8, 1),
                                             (8_810, 64, 3), (10, 8, 3)])
def test_resharded_read_matches_flat_slices(tmp_path, psi, n_old, n_new):
    flat = state(psi, 11)
    paths = []
    for k in range(n_old):
        lay = oracle.layout(psi, n_old, k)
        sl = slice(lay.offset, lay.offset + lay.count)
        p = str(tmp_path / f"old{k}.zshard")
        zs.zero_ckpt_write(p, psi, n_old, k, "f16", zs.Scaler(8.0),
                           *(np.ascontiguousarray(a[sl]) for a in flat))
        paths.append(p)
    for r in range(n_new):
        lay = oracle.layout(psi, n_new, r)
        got = zs.zero_ckpt_read_resharded(paths, psi, n_new, r)
        for a, b in zip(flat, got):
            assert np.array_equal(a[lay.offset:lay.offset + lay.count].view(np.uint8),
                                  b.view(np.uint8))


def test_resume_on_another_rank_count_is_exact(tmp_path):
    # oracle-level invariant: 3 steps on 8 shards, save, resume on 5 shards,
    # 2 more steps == 5 steps on the unsharded buffer
    psi = 50_021
    rng = np.random.default_rng(21)
    grads = [(rng.standard_normal(psi) * 1e-3).astype(np.float16).view(np.uint16)
             for _ in range(5)]
    master0 = (rng.standard_normal(psi) * 0.02).astype(np.float32)
    full = [np.zeros(psi, np.uint16), master0.copy(), np.zeros(psi, np.float32),
            np.zeros(psi, np.float32)]
    for t in range(1, 6):
        oracle.adam_step(full[0], grads[t - 1], full[1], full[2], full[3], "f16", step=t,
                         loss_scale=1.0, **HP)
    paths = []
    for k in range(8):
        lay = oracle.layout(psi, 8, k)
        sl = slice(lay.offset, lay.offset + lay.count)
        sh = [np.zeros(lay.count, np.uint16), master0[sl].copy(),
              np.zeros(lay.count, np.float32), np.zeros(lay.count, np.float32)]
        for t in range(1, 4):
            oracle.adam_step(sh[0], np.ascontiguousarray(grads[t - 1][sl]), sh[1], sh[2], sh[3],
                             "f16", step=t, loss_scale=1.0, **HP)
        p = str(tmp_path / f"k{k}.zshard")
        zs.zero_ckpt_write(p, psi, 8, k, "f16", zs.Scaler(1.0, step=3), *sh)
        paths.append(p)
    for r in range(5):
        lay = oracle.layout(psi, 5, r)
        sl = slice(lay.offset, lay.offset + lay.count)
        sh = list(zs.zero_ckpt_read_resharded(paths, psi, 5, r))
        t0 = zs.zero_ckpt_read_info(paths[0]).scaler.step
        for t in range(t0 + 1, t0 + 3):
            oracle.adam_step(sh[0], np.ascontiguousarray(grads[t - 1][sl]), sh[1], sh[2], sh[3],
                             "f16", step=t, loss_scale=1.0, **HP)
        for a, b in zip(full, sh):
            assert np.array_equal(a[sl].view(np.uint8), b.view(np.uint8))


def test_resharded_read_refuses_mixed_steps_and_bad_payloads(tmp_path):
    # a save that failed part-way leaves rank 1's file one step behind; every
    # new rank must refuse the set (also new rank 0, which reads only old file 0)
    psi, n_old, n_new = 40_009, 4, 2
    flat = state(psi, 5)
    paths = []
    for k in range(n_old):
        lay = oracle.layout(psi, n_old, k)
        sl = slice(lay.offset, lay.offset + lay.count)
        p = str(tmp_path / f"s{k}.zshard")
        zs.zero_ckpt_write(p, psi, n_old, k, "f16", zs.Scaler(1024.0, step=10),
                           *(np.ascontiguousarray(a[sl]) for a in flat))
        paths.append(p)
    for r in range(n_new):
        zs.zero_ckpt_read_resharded(paths, psi, n_new, r)           # consistent: reads
    lay1 = oracle.layout(psi, n_old, 1)
    sl1 = slice(lay1.offset, lay1.offset + lay1.count)
    stale = zs.Scaler(1024.0, step=9)
    zs.zero_ckpt_write(paths[1], psi, n_old, 1, "f16", stale,
                       *(np.ascontiguousarray(a[sl1]) for a in flat))
    for r in range(n_new):
        with pytest.raises(zs.ZeroError) as e:
            zs.zero_ckpt_read_resharded(paths, psi, n_new, r)
        assert e.value.code == -6, r
    # other scaler fields and the format must agree too
    for sc, dt in ((zs.Scaler(2048.0, step=10), "f16"), (zs.Scaler(1024.0, step=10), "bf16"),
                   (zs.Scaler(1024.0, growth_interval=7, step=10), "f16")):
        zs.zero_ckpt_write(paths[1], psi, n_old, 1, dt, sc,
                           *(np.ascontiguousarray(a[sl1]) for a in flat))
        with pytest.raises(zs.ZeroError) as e:
            zs.zero_ckpt_read_resharded(paths, psi, n_new, 0)
        assert e.value.code == -6, (sc.loss_scale, dt)
    sc = zs.Scaler(1024.0, step=10)
    zs.zero_ckpt_write(paths[1], psi, n_old, 1, "f16", sc,
                       *(np.ascontiguousarray(a[sl1]) for a in flat))
    zs.zero_ckpt_read_resharded(paths, psi, n_new, 0)               # whole again
    # a flipped payload byte in a file the new rank reads is caught by its hash
    raw = bytearray(open(paths[3], "rb").read())
    raw[128 + 777] ^= 0x01
    open(paths[3], "wb").write(bytes(raw))
    zs.zero_ckpt_read_resharded(paths, psi, n_new, 0)               # reads old files 0-1 only
    with pytest.raises(zs.ZeroError) as e:
        zs.zero_ckpt_read_resharded(paths, psi, n_new, 1)           # reads old files 2-3
    assert e.value.code == -6
    # a missing old file is an argument error for every new rank
    with pytest.raises((zs.ZeroError, TypeError, ValueError)):
        zs.zero_ckpt_read_resharded(paths[:3] + [None], psi, n_new, 0)
