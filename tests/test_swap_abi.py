"""CPU tests of the host tier through the C ABI: the library's swap bookkeeping
agrees bit for bit with the oracle's (pairs, free lists of both tiers,
residency of every table entry, reference counts) on the tool-pause workload
and on random programs; refused requests change nothing; deferred frames and
blocks wait for their fence.  Pools and host tiers are created over NULL
buffers: no device work is done here.
"""

import numpy as np
import pytest

from oracle import footprint
from oracle.block_manager import BlockManager
from pagedattention_decode_amd import binding as B
from pagedattention_decode_amd.pool import PagedKVPool
from synth import draws, workloads


def host_pool(args, free_order=None):
    return PagedKVPool(*args, free_order=free_order, allocate=False)


def assert_same(pool, bm, n_frames):
    assert list(pool.free_list()) == list(bm.free)
    assert list(pool.refcounts()) == bm.ref
    assert list(pool.host_free_list()) == list(bm.host_free)
    for s in bm.tables:
        tiers, idx = pool.residency(s)
        expect = bm.residency(s)
        assert [("host" if t == B.KV_TIER_HOST else "hbm", int(i)) for t, i in zip(tiers, idx)] == expect, s
        assert pool.info(s) == (bm.lengths[s], len(expect))
    pool.check()
    bm.check()


def test_frame_bytes_is_a_block_of_every_layer():
    # the pages' 70B shape: one frame is B tokens of the per-token footprint
    pool = host_pool((80, 4, 16, 8, 128, "bf16"))
    assert B.kv_host_frame_bytes(pool.handle) == footprint.block_bytes(80, 8, 16, 128, 2) == 16 * 327680
    for fmt, bits in (("q8_0", 8), ("q4_0", 4)):
        q = host_pool((3, 4, 16, 2, 64, fmt))
        tile = 16 * 64 * bits // 8 + 16 * 64 // 32 * 2
        assert B.kv_host_frame_bytes(q.handle) == 2 * 3 * 2 * tile


def replay_tool_pause():
    wl = workloads.tool_pause(layers=1)
    order = draws.free_order(wl.seed, wl.num_blocks)
    pool = host_pool((wl.num_layers, wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim, wl.dtype), order)
    bm = BlockManager(wl.num_blocks, wl.block_size, order)
    n_frames = None
    swaps = 0
    for op in wl.ops:
        kind = op[0]
        if kind == "host":
            n_frames = op[1]
            horder = None if len(op) > 2 else draws.host_free_order(wl.seed, n_frames)
            pool.attach_host(n_frames, horder)
            bm.attach_host(n_frames, horder)
        elif kind == "add":
            pool.add(op[1]); bm.add(op[1])
        elif kind == "fork":
            pool.fork(op[1], op[2]); bm.fork(op[1], op[2])
        elif kind == "append":
            slots, pairs = pool.append(op[1], op[2])
            r_slots, r_pairs = bm.append(op[1], op[2])
            assert np.array_equal(slots, np.asarray(r_slots, np.int64))
            assert [tuple(p) for p in pairs.tolist()] == r_pairs
        elif kind == "swap_out":
            got = pool.swap_out_fenced(op[1], 0)
            assert [tuple(p) for p in got.tolist()] == bm.swap_out(op[1])
            swaps += 1
        elif kind == "swap_in":
            got = pool.swap_in_fenced(op[1], 0)
            assert [tuple(p) for p in got.tolist()] == bm.swap_in(op[1])
            swaps += 1
        elif kind == "decode":
            pass
        else:
            raise ValueError(kind)
        if n_frames:
            assert_same(pool, bm, n_frames)
    assert swaps == 4
    return pool, bm


def test_tool_pause_bookkeeping_bit_exact():
    replay_tool_pause()


def test_swapped_sequences_are_refused_by_readers_and_writers():
    pool = host_pool((1, 16, 4, 1, 32, "bf16"))
    pool.attach_host(8)
    pool.add(0)
    pool.append([0], [9])
    pool.add(1)
    pool.append([1], [3])
    assert len(pool.swap_out_fenced(0, 0)) == 3
    for call in (lambda: pool.append([0], [1]), lambda: pool.fork(0, 5), lambda: pool.tables([0], 8),
                 lambda: pool.shared_prefix_plan([1, 0]), lambda: pool.prefix_insert(0, list(range(9))),
                 lambda: pool.swap_out_fenced(0, 0)):
        with pytest.raises(B.KVError) as e:
            call()
        assert e.value.status == B.KV_ERR_INVALID
    # others are unaffected; release of a swapped sequence gives its frames back
    pool.append([1], [1])
    assert list(pool.host_free_list()) == [3, 4, 5, 6, 7]
    pool.release_fenced(0, 0)
    assert list(pool.host_free_list()) == [3, 4, 5, 6, 7, 0, 1, 2]
    pool.check()
    # the device side refuses a pool without memory, before touching a stream
    with pytest.raises(B.KVError) as e:
        pool.swap_copy([[0, 0]], 0, stream=0)
    assert e.value.status == B.KV_ERR_INVALID
    with pytest.raises(B.KVError):
        pool.swap_out(1, stream=0)


def test_refused_swaps_change_nothing():
    pool = host_pool((2, 6, 4, 1, 32, "bf16"), list(range(6)))
    bm = BlockManager(6, 4, list(range(6)))
    pool.attach_host(2); bm.attach_host(2)
    for x in (pool, bm):
        x.add(0)
        x.append([0], [12])
    with pytest.raises(B.KVOutOfBlocks):
        pool.swap_out_fenced(0, 0)
    with pytest.raises(MemoryError):
        bm.swap_out(0)
    assert_same(pool, bm, 2)
    for x in (pool, bm):
        x.add(1)
        x.append([1], [8])
    assert pool.swap_out_fenced(1, 0).tolist() == [list(p) for p in bm.swap_out(1)]
    for x in (pool, bm):
        x.add(2)
        x.append([2], [12])
    with pytest.raises(B.KVOutOfBlocks):
        pool.swap_in_fenced(1, 0)
    with pytest.raises(MemoryError):
        bm.swap_in(1)
    assert_same(pool, bm, 2)


def test_deferred_blocks_and_frames_wait_for_their_fence():
    pool = host_pool((1, 8, 4, 1, 32, "bf16"), list(range(8)))
    pool.attach_host(4)
    pool.add(0)
    pool.append([0], [8])                        # blocks 0, 1
    assert pool.swap_out_fenced(0, 5).tolist() == [[0, 0], [1, 1]]
    assert 0 not in pool.free_list() and pool.stats()["n_pending"] == 2
    pool.retire(4)
    assert 0 not in pool.free_list()
    pool.retire(5)
    assert list(pool.free_list())[-2:] == [0, 1]
    pairs = pool.swap_in_fenced(0, 9)             # frames 0, 1 wait for fence 9
    assert pairs[:, 0].tolist() == [0, 1]
    assert list(pool.host_free_list()) == [2, 3]
    pool.retire(9)
    assert list(pool.host_free_list()) == [2, 3, 0, 1]
    pool.check()


@pytest.mark.parametrize("seed", range(8))
def test_random_swap_programs_bit_exact(seed):
    rng = np.random.default_rng(seed)
    Bs = int(rng.choice([1, 2, 4, 16]))
    N = int(rng.integers(6, 40))
    F = int(rng.integers(3, 24))
    order = rng.permutation(N).astype(np.int32)
    horder = rng.permutation(F).astype(np.int32)
    pool = host_pool((1, N, Bs, 1, 32, "bf16"), order)
    bm = BlockManager(N, Bs, order)
    pool.attach_host(F, horder)
    bm.attach_host(F, horder)
    live, nxt = [], 0
    n_swaps = 0
    for _ in range(250):
        op = rng.random()
        resident = [s for s in live if not bm.swapped(s)]
        swapped = [s for s in live if bm.swapped(s)]
        if op < 0.15 or not live:
            pool.add(nxt); bm.add(nxt); live.append(nxt); nxt += 1
        elif op < 0.45 and resident:
            s = int(rng.choice(resident)); c = int(rng.integers(0, 3 * Bs))
            try:
                r = bm.append([s], [c])
            except MemoryError:
                with pytest.raises(B.KVOutOfBlocks):
                    pool.append([s], [c])
            else:
                slots, pairs = pool.append([s], [c])
                assert [tuple(p) for p in pairs.tolist()] == r[1]
        elif op < 0.55 and resident:
            s = int(rng.choice(resident))
            pool.fork(s, nxt); bm.fork(s, nxt); live.append(nxt); nxt += 1
        elif op < 0.7 and resident:
            s = int(rng.choice(resident))
            try:
                r = bm.swap_out(s)
            except MemoryError:
                with pytest.raises(B.KVOutOfBlocks):
                    pool.swap_out_fenced(s, 0)
            else:
                assert [tuple(p) for p in pool.swap_out_fenced(s, 0).tolist()] == r
                n_swaps += 1
        elif op < 0.85 and swapped:
            s = int(rng.choice(swapped))
            try:
                r = bm.swap_in(s)
            except MemoryError:
                with pytest.raises(B.KVOutOfBlocks):
                    pool.swap_in_fenced(s, 0)
            else:
                assert [tuple(p) for p in pool.swap_in_fenced(s, 0).tolist()] == r
                n_swaps += 1
        elif live:
            s = int(rng.choice(live))
            pool.release_fenced(s, 0); bm.release(s); live.remove(s)
        assert_same(pool, bm, F)
    assert n_swaps >= 6
