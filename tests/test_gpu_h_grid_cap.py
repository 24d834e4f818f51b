"""The tile loops of the streaming kernels, driven at small sizes.

A shard with more tiles than the launch has blocks (beyond 2^23 blocks, about
1.7e10 elements for the step) is walked by each block in turn.  Such shards do
not fit in one GPU's memory with the step's five arrays, so these tests lower
the grid cap with zero_set_grid_cap to 1, 3 and 7 blocks and check every
kernel against the oracle at sizes of many tiles with ragged heads and tails:
the step (vector and element-wise paths, 16-bit and FP32 gradients), the
accumulate, the flag check and both exchanges.  The occupancy setting
(zero_set_occupancy) must leave every result bit and flag unchanged.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import zero_sharded_mixed_shard_amd as zs
from gpu_util import GuardedView, SENT16, assert_close, f32, log, u16
from test_gpu_a_small import run_case
from test_gpu_d_g32 import HP, TD, micro_batches
from test_gpu_e_exchange import host, make_replicas

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
CAPS = (1, 3, 7)
COUNTS = (11_017, 40_965)     # 5 and 20 step tiles, with ragged tails


@pytest.fixture(params=CAPS)
def cap(request):
    zs.zero_set_grid_cap(request.param)
    yield request.param
    torch.cuda.synchronize()
    zs.zero_set_grid_cap(0)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_step_tile_loop(cap, dtype):
    for count in COUNTS:
        for phase in (0, 3):
            run_case(count, dtype, dict.fromkeys(("g16", "w16", "master", "m", "v"), phase),
                     steps=2, seed=count + phase)
        # views of different phases: the element-wise kernel's grid-stride loop
        run_case(count, dtype, dict(g16=1, w16=2, master=0, m=3, v=1), steps=2, seed=count)
    log(f"step {dtype} cap {cap}: within the bar")


def test_step_g32_and_accumulate_tile_loop(cap):
    g32_and_accumulate_case(f"cap={cap}", cap)


def g32_and_accumulate_case(label, seed):
    rng = np.random.default_rng(seed)
    for count in COUNTS:
        for dtype in ("f16", "bf16"):
            acc = GuardedView(count, torch.float32, 1, DEV)
            gv = GuardedView(count, TD[dtype], 1, DEV)
            ref_acc = np.zeros(count, np.float32)
            flag = torch.full((1,), 7, dtype=torch.int32, device=DEV)
            mbs = micro_batches(count, 3, dtype, 70 + seed)
            for j, g in enumerate(mbs):
                gv.view.copy_(g.to(DEV))
                if j == len(mbs) - 1:      # the last one with the fused FP32 check
                    zs.zero_grad_accumulate_check(acc.view, gv.view, count, 1, 0, first=(j == 0),
                                                  loss_scale=3.0, found_inf=flag)
                else:
                    zs.zero_grad_accumulate(acc.view, gv.view, count, 1, 0, first=(j == 0))
                oracle.grad_accumulate(ref_acc, u16(g), dtype, first=(j == 0))
            torch.cuda.synchronize()
            assert np.array_equal(f32(acc.view).view(np.uint32), ref_acc.view(np.uint32))
            assert flag.item() == oracle.overflow_check_g32(ref_acc, 3.0)[0] == 0
            assert acc.guards_intact() and gv.guards_intact()

            V = {k: GuardedView(count, torch.float32, 2, DEV) for k in ("master", "m", "v")}
            V["w16"] = GuardedView(count, TD[dtype], 2, DEV)
            master0 = (rng.standard_normal(count) * 0.02).astype(np.float32)
            V["master"].view.copy_(torch.from_numpy(master0).to(DEV))
            for k in ("m", "v", "w16"):
                V[k].view.zero_()
            ref = dict(master=master0.copy(), m=np.zeros(count, np.float32),
                       v=np.zeros(count, np.float32), w16=np.zeros(count, np.uint16))
            G = GuardedView(count, torch.float32, 2, DEV)
            for t in (1, 2):
                g = (rng.standard_normal(count) * 1e-3).astype(np.float32)
                G.view.copy_(torch.from_numpy(g).to(DEV))
                zs.zero_adam_step_g32(V["w16"].view, G.view, V["master"].view, V["m"].view,
                                      V["v"].view, count, 1, 0, step=t, loss_scale=1.0, **HP)
                oracle.adam_step_g32(ref["w16"], g, ref["master"], ref["m"], ref["v"], dtype,
                                     step=t, loss_scale=1.0, **HP)
            torch.cuda.synchronize()
            got = dict(master=f32(V["master"].view), m=f32(V["m"].view), v=f32(V["v"].view),
                       w16=u16(V["w16"].view))
            assert_close(got, ref, dtype, f"g32 {label} count={count}")
            assert all(x.guards_intact() for x in list(V.values()) + [G])


# Elements per launch of the step and the accumulates: below one tile (one
# tile per launch), three tiles and a remainder (rounded down to three), and
# seven tiles.  The shard goes out as consecutive launches; every result bit
# must match the oracle, heads, tails and the element-wise path included.
PIECES = (1, 3 * 2048 + 5, 7 * 2048)


@pytest.fixture(params=PIECES)
def piece(request):
    zs.zero_set_launch_piece(request.param)
    yield request.param
    torch.cuda.synchronize()
    zs.zero_set_launch_piece(0)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_step_in_pieces(piece, dtype):
    for count in COUNTS:
        for phase in (0, 3):
            run_case(count, dtype, dict.fromkeys(("g16", "w16", "master", "m", "v"), phase),
                     steps=2, seed=count + phase + 7)
        run_case(count, dtype, dict(g16=1, w16=2, master=0, m=3, v=1), steps=2, seed=count + 7)
    log(f"step {dtype} in pieces of {piece}: within the bar")


def test_step_g32_and_accumulate_in_pieces(piece):
    g32_and_accumulate_case(f"piece={piece}", piece % 97)


@pytest.mark.parametrize("fmt", ["f16", "bf16", "f32"])
def test_flag_check_in_pieces(fmt):
    # the flag-only check cut into launches of one, three or seven tiles of
    # 1024 vectors: a non-finite value at the head, at either side of a piece
    # boundary, inside the last partial tile and in the elements after the
    # last vector is seen, and a clean buffer leaves the flag 0
    td = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[fmt]
    per = 4 if fmt == "f32" else 8
    tile = 1024 * per
    count = 9 * tile + 3 * per + 5
    g = synth.fill_normal_(torch.empty(count, dtype=td), 1e-3, 81)
    gv = GuardedView(count, td, 3, DEV)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    check = zs.zero_overflow_check_g32 if fmt == "f32" else zs.zero_overflow_check
    try:
        for piece in PIECES:
            zs.zero_set_launch_piece(piece * per // 2)   # 1, 3 and 7 tiles of this format
            gv.view.copy_(g.to(DEV))
            check(gv.view, count, 1, 0, 1024.0, flag)
            assert int(flag.item()) == 0, (fmt, piece)
            for pos in (0, 2, tile - 1, tile, 3 * tile - 1, 3 * tile + 1, 7 * tile, 9 * tile + 7,
                        count - 1):
                bad = g.clone()
                bad[pos] = float("inf") if pos % 2 else float("nan")
                gv.view.copy_(bad.to(DEV))
                check(gv.view, count, 1, 0, 1024.0, flag)
                want = (oracle.overflow_check_g32(f32(bad), 1024.0)[0] if fmt == "f32"
                        else oracle.overflow_check(u16(bad), fmt, 1024.0)[0])
                assert int(flag.item()) == want == 1, (fmt, piece, pos)
    finally:
        torch.cuda.synchronize()
        zs.zero_set_launch_piece(0)
    assert gv.guards_intact()
    log(f"flag check {fmt} in pieces of 1, 3 and 7 tiles: every planted value seen")


def test_pieces_with_a_lowered_grid_cap():
    # both overrides at once: launches of seven tiles, each walked by three
    # blocks in turn (the tile loop inside every piece)
    zs.zero_set_launch_piece(7 * 2048)
    zs.zero_set_grid_cap(3)
    try:
        for dtype in ("f16", "bf16"):
            for count in COUNTS:
                run_case(count, dtype, dict.fromkeys(("g16", "w16", "master", "m", "v"), 3),
                         steps=2, seed=count + 11)
        g32_and_accumulate_case("piece=7 tiles, cap=3", 13)
    finally:
        torch.cuda.synchronize()
        zs.zero_set_grid_cap(0)
        zs.zero_set_launch_piece(0)
    log("pieces of seven tiles under a grid cap of three blocks: within the bar")


def test_flag_tile_loop(cap):
    count = 200_003
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    g = synth.fill_normal_(torch.empty(count, dtype=torch.float16), 1e-3, 5)
    gv = GuardedView(count, torch.float16, 3, DEV)
    gv.view.copy_(g.to(DEV))
    zs.zero_overflow_check(gv.view, count, 1, 0, 1024.0, flag)
    assert flag.item() == 0
    for pos in (0, 1, count // 2, count - 9, count - 1):
        bad = g.clone()
        bad[pos] = float("nan") if pos % 2 else float("inf")
        gv.view.copy_(bad.to(DEV))
        zs.zero_overflow_check(gv.view, count, 1, 0, 1024.0, flag)
        assert flag.item() == oracle.overflow_check(u16(bad), "f16", 1024.0)[0] == 1, pos
    x = torch.zeros(count, device=DEV)
    x[count - 1] = float("inf")
    zs.zero_overflow_check_g32(x, count, 1, 0, 1.0, flag)
    assert flag.item() == 1
    assert gv.guards_intact()


def test_exchanges_tile_loop(cap):
    for psi, n, phase in ((50_003, 3, 0), (50_003, 3, 1), (131_077, 4, 0)):
        reps = make_replicas(psi, n, "f16", psi + n + cap, phase)
        hreps = [host(r) for r in reps]
        shards = []
        for k in range(n):
            lay = zs.zero_shard_layout(psi, n, k)
            out = torch.empty(lay.count + 8, dtype=torch.float16, device=DEV)[phase:phase + lay.count]
            zs.zero_reduce_shard(out, reps, psi, n, k)
            ref = oracle.reduce_shard(hreps, "f16", "f16", psi, n, k)
            assert np.array_equal(u16(out), ref), (psi, n, k, phase)
            shards.append(out)
        full = GuardedView(zs.zero_shard_layout(psi, n, 0).padded_total, torch.float16, 0, DEV)
        zs.zero_gather_shards(full.view, shards, psi, n)
        got = u16(full.view)
        want = np.zeros(psi, np.uint16)
        oracle.gather_shards([u16(s) for s in shards], psi, n, want)
        assert np.array_equal(got[:psi], want)
        assert np.all(got[psi:] == SENT16) and full.guards_intact()
    log(f"exchanges cap {cap}: bitwise")


def test_step_occupancy_settings_change_nothing():
    # The step's occupancy cap is an LDS reservation the kernel never touches:
    # under every setting -- the kernel's rule (0; 2 per CU), 1, 2, 3 and no
    # cap (8) -- the same inputs give the same bits, and windows match the
    # oracle.  2^28 + 12,345 elements at phase 3, both formats.
    count, phase = (1 << 28) + 12_345, 3
    for dtype in ("f16", "bf16"):
        td = TD[dtype]
        g16 = synth.fill_normal_(torch.empty(count, dtype=td), 1e-3, 71_000)
        master0 = synth.fill_normal_(torch.empty(count), 0.02, 71_001)
        V = {k: GuardedView(count, td if k in ("g16", "w16") else torch.float32, phase, DEV)
             for k in ("g16", "w16", "master", "m", "v")}
        V["g16"].view.copy_(g16.to(DEV))
        results = {}
        try:
            for occ in (0, 1, 2, 3, 8):
                zs.zero_set_occupancy(occ)
                V["master"].view.copy_(master0.to(DEV))
                for k in ("m", "v", "w16"):
                    V[k].view.zero_()
                for t in (1, 2):
                    zs.zero_adam_step(V["w16"].view, V["g16"].view, V["master"].view,
                                      V["m"].view, V["v"].view, count, 1, 0, step=t,
                                      loss_scale=1024.0, **HP)
                torch.cuda.synchronize()
                results[occ] = {k: V[k].view.clone() for k in ("w16", "master", "m", "v")}
        finally:
            torch.cuda.synchronize()
            zs.zero_set_occupancy(0)
        for occ in (1, 2, 3, 8):
            for k in results[0]:
                assert torch.equal(results[occ][k].view(torch.int16 if k == "w16" else
                                                        torch.int32),
                                   results[0][k].view(torch.int16 if k == "w16" else
                                                      torch.int32)), (dtype, occ, k)
        assert all(v.guards_intact() for v in V.values())
        wins = [(0, 4096), (count // 2, count // 2 + 4096), (count - 4096, count)]
        gh = u16(g16)
        for a, b in wins:
            ref = dict(master=master0[a:b].numpy().copy(), m=np.zeros(b - a, np.float32),
                       v=np.zeros(b - a, np.float32), w16=np.zeros(b - a, np.uint16))
            for t in (1, 2):
                oracle.adam_step(ref["w16"], gh[a:b], ref["master"], ref["m"], ref["v"], dtype,
                                 step=t, loss_scale=1024.0, **HP)
            got = {k: (u16 if k == "w16" else f32)(results[0][k][a:b]) for k in ref}
            assert_close(got, ref, dtype, f"occupancy window {a}")
        del results, V
        torch.cuda.empty_cache()
    log("step occupancy settings 0/1/2/3/8: bitwise equal, windows match the oracle")


def test_step_launch_pieces_change_nothing():
    # The step's own rule splits a shard past 2^27 elements into launches of
    # 2^27 (here three and a ragged fourth): the default, one launch over
    # everything, and pieces of 3 * 2^20 + 7 elements give the same bits, and
    # windows across piece boundaries match the oracle.  2^28 + 2^27 + 12,345
    # elements at phase 3, FP16.
    count, phase, dtype = (1 << 28) + (1 << 27) + 12_345, 3, "f16"
    td = TD[dtype]
    g16 = synth.fill_normal_(torch.empty(count, dtype=td), 1e-3, 73_000)
    master0 = synth.fill_normal_(torch.empty(count), 0.02, 73_001)
    V = {k: GuardedView(count, td if k in ("g16", "w16") else torch.float32, phase, DEV)
         for k in ("g16", "w16", "master", "m", "v")}
    V["g16"].view.copy_(g16.to(DEV))
    results = {}
    try:
        for piece in (0, 2 ** 64 - 1, 3 * (1 << 20) + 7):
            zs.zero_set_launch_piece(piece)
            V["master"].view.copy_(master0.to(DEV))
            for k in ("m", "v", "w16"):
                V[k].view.zero_()
            for t in (1, 2):
                zs.zero_adam_step(V["w16"].view, V["g16"].view, V["master"].view, V["m"].view,
                                  V["v"].view, count, 1, 0, step=t, loss_scale=1000.0, **HP)
            torch.cuda.synchronize()
            results[piece] = {k: V[k].view.clone() for k in ("w16", "master", "m", "v")}
    finally:
        torch.cuda.synchronize()
        zs.zero_set_launch_piece(0)
    for piece in list(results)[1:]:
        for k in results[0]:
            iv = torch.int16 if k == "w16" else torch.int32
            assert torch.equal(results[piece][k].view(iv), results[0][k].view(iv)), (piece, k)
    assert all(v.guards_intact() for v in V.values())
    gh = u16(g16)
    b28 = 1 << 28
    for a, b in ((0, 4096), (b28 - 4096, b28 + 4096), (count - 4096, count)):
        ref = dict(master=master0[a:b].numpy().copy(), m=np.zeros(b - a, np.float32),
                   v=np.zeros(b - a, np.float32), w16=np.zeros(b - a, np.uint16))
        for t in (1, 2):
            oracle.adam_step(ref["w16"], gh[a:b], ref["master"], ref["m"], ref["v"], dtype,
                             step=t, loss_scale=1000.0, **HP)
        got = {k: (u16 if k == "w16" else f32)(results[0][k][a:b]) for k in ref}
        assert_close(got, ref, dtype, f"piece window {a}")
    del results, V
    torch.cuda.empty_cache()
    log("step launch pieces default/one/3M+7: bitwise equal, windows match the oracle")


def test_accumulate_and_check_occupancy_settings_change_nothing():
    # The same for the accumulates (first micro-batch, later ones, the fused
    # check) and the flag-only check: every setting gives the same bits and
    # flags.  2^28 + 777 elements (past the size where the rules cap) at phase 1,
    # with one non-finite gradient planted for the flags.
    count, phase = (1 << 28) + 777, 1
    g16 = synth.fill_normal_(torch.empty(count, dtype=torch.float16), 1e-3, 72_000)
    g16b = synth.fill_normal_(torch.empty(count, dtype=torch.float16), 1e-3, 72_001)
    g16b[count - 5] = float("inf")
    G = GuardedView(count, torch.float16, phase, DEV)
    Gb = GuardedView(count, torch.float16, phase, DEV)
    G.view.copy_(g16.to(DEV))
    Gb.view.copy_(g16b.to(DEV))
    A = GuardedView(count, torch.float32, phase, DEV)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    results = {}
    try:
        for occ in (0, 1, 2, 4, 8):
            zs.zero_set_occupancy(occ)
            flags = []
            zs.zero_grad_accumulate(A.view, G.view, count, 1, 0, first=True)
            zs.zero_grad_accumulate(A.view, G.view, count, 1, 0, first=False)
            zs.zero_grad_accumulate_check(A.view, Gb.view, count, 1, 0, first=False,
                                          loss_scale=1024.0, found_inf=flag)
            flags.append(int(flag.item()))
            for g in (G, Gb):
                zs.zero_overflow_check(g.view, count, 1, 0, 1024.0, flag)
                flags.append(int(flag.item()))
            torch.cuda.synchronize()
            results[occ] = (A.view.clone(), flags)
    finally:
        torch.cuda.synchronize()
        zs.zero_set_occupancy(0)
    assert results[0][1] == [1, 0, 1]
    for occ in (1, 2, 4, 8):
        assert results[occ][1] == results[0][1], occ
        assert torch.equal(results[occ][0].view(torch.int32), results[0][0].view(torch.int32)), occ
    assert A.guards_intact() and G.guards_intact() and Gb.guards_intact()
    # two windows against the oracle's accumulate
    for a, b in ((0, 4096), (count - 4096, count)):
        acc = np.zeros(b - a, np.float32)
        oracle.grad_accumulate(acc, u16(g16)[a:b], "f16", True)
        oracle.grad_accumulate(acc, u16(g16)[a:b], "f16", False)
        oracle.grad_accumulate(acc, u16(g16b)[a:b], "f16", False)
        assert np.array_equal(f32(results[0][0][a:b]).view(np.uint32), acc.view(np.uint32))
    del results
    torch.cuda.empty_cache()
    log("accumulate / check occupancy settings 0/1/2/4/8: bitwise equal flags and sums")


def test_exchange_occupancy_settings_change_nothing():
    # the reduce and the gather under every occupancy setting: the same bits
    psi, n = 3 * (1 << 20) + 101, 4
    reps = [synth.fill_normal_(torch.empty(psi, dtype=torch.float16, device=DEV), 1e-2,
                               73_000 + k) for k in range(n)]
    lay = zs.zero_shard_layout(psi, n, 1)
    shards = [r[:zs.zero_shard_layout(psi, n, k).count].clone() for k, r in enumerate(reps)]
    results = {}
    try:
        for occ in (0, 1, 2, 4, 8):
            zs.zero_set_occupancy(occ)
            out = torch.empty(lay.count, dtype=torch.float16, device=DEV)
            full = torch.zeros(psi, dtype=torch.float16, device=DEV)
            zs.zero_reduce_shard(out, reps, psi, n, 1)
            zs.zero_gather_shards(full, shards, psi, n)
            torch.cuda.synchronize()
            results[occ] = (out, full)
    finally:
        torch.cuda.synchronize()
        zs.zero_set_occupancy(0)
    for occ in (1, 2, 4, 8):
        for a, b in zip(results[occ], results[0]):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), occ
    want = oracle.reduce_shard([u16(r) for r in reps], "f16", "f16", psi, n, 1)
    assert np.array_equal(u16(results[0][0]), want)
    log("exchange occupancy settings 0/1/2/4/8: bitwise equal, reduce equals the oracle")
