"""Pins of the oracle's host tier (block swap to pinned host memory).

[KVM] asynchronous paged swap (Figure 11, the three migration steps) and the
evict-versus-swap analysis with its worked estimate for a 45-second tool wait.
The oracle is checked against the numbers the pages print, against its
conservation invariant on random programs, and against what a swap must not
change: the bytes of every block, the blocks other holders share, and the
state after a refused (all-or-nothing) request.
"""

import copy
import math
import random

import numpy as np
import pytest

from oracle import footprint
from oracle.block_manager import BlockManager
from oracle.kv_store import KVStore
from oracle.runner import OracleReplay
from synth import workloads


# ---------------------------------------------------------------------------
# the pages' numbers
# ---------------------------------------------------------------------------

def test_worked_estimate_of_a_paused_agent():
    """[KVM] estimate for a 70B model paused at 32768 tokens: 10.7 GB of KV, 21 ms to reload
    over 8 links of 64 GB/s (42 ms round trip), 4.63e15 operations and 1.3 s to recompute at
    3560 TFLOP/s, so reloading is about 62x faster.  The 70B shape is 80 layers, 8 KV heads,
    d = 128, 2-byte elements (the same model's 5.0 GiB at 16384 tokens, Figure 10)."""
    m_token = footprint.kv_bytes_per_token(80, 8, 128, 2)
    assert m_token == 327680
    assert round(32768 * m_token / 1e9, 1) == 10.7
    assert 16384 * m_token == 5 * 2 ** 30
    reload = footprint.reload_seconds(32768, m_token, 512e9)
    assert round(reload * 1e3) == 21 and round(2 * reload * 1e3) == 42
    assert round(2 * 70.6e9 * 32768 / 1e15, 2) == 4.63
    recompute = footprint.recompute_seconds(70.6e9, 32768, 3560e12)
    assert round(recompute, 1) == 1.3
    assert round(recompute / reload) == 62
    # one host frame holds one block of every layer: B tokens of m_token bytes
    assert footprint.block_bytes(80, 8, 16, 128, 2) == 16 * m_token


# ---------------------------------------------------------------------------
# bookkeeping
# ---------------------------------------------------------------------------

def state(bm):
    return (list(bm.free), list(bm.ref), {s: list(t) for s, t in bm.tables.items()}, dict(bm.lengths),
            list(bm.host_free), copy.deepcopy(bm.frames))


def test_swap_out_moves_only_exclusive_blocks_fifo():
    bm = BlockManager(12, 4, list(range(12)))
    bm.attach_host(5, [4, 3, 2, 1, 0])
    bm.add(0)
    bm.append([0], [10])          # blocks 0, 1, 2 (2 partly filled)
    bm.fork(0, 1)                 # all three shared
    bm.append([1], [1])           # 1 copies the partly filled block 2 -> 3
    assert bm.table(0) == [0, 1, 2] and bm.table(1) == [0, 1, 3]
    pairs = bm.swap_out(0)
    assert pairs == [(2, 4)]      # only block 2 is held by 0 alone; frames from the front
    assert bm.residency(0) == [("hbm", 0), ("hbm", 1), ("host", 4)]
    assert list(bm.free)[-1] == 2 and bm.ref[2] == 0 and bm.ref[0] == 2
    assert list(bm.host_free) == [3, 2, 1, 0]
    bm.check()
    with pytest.raises(ValueError):
        bm.append([0], [1])
    with pytest.raises(ValueError):
        bm.fork(0, 2)
    with pytest.raises(ValueError):
        bm.table(0)
    # swap-in pops from the front of the free list, frames go to the back of theirs
    front = bm.free[0]
    assert bm.swap_in(0) == [(4, front)]
    assert bm.table(0) == [0, 1, front] and list(bm.host_free) == [3, 2, 1, 0, 4]
    bm.check()


def test_release_of_a_swapped_sequence_returns_frames_in_table_order():
    bm = BlockManager(16, 2, list(range(16)))
    bm.attach_host(8)
    bm.add(7)
    bm.append([7], [7])           # blocks 0..3
    assert bm.swap_out(7) == [(0, 0), (1, 1), (2, 2), (3, 3)]
    assert bm.release(7) == []
    assert list(bm.host_free) == [4, 5, 6, 7, 0, 1, 2, 3]
    assert bm.n_free() == 16
    bm.check()


def test_refused_requests_change_nothing():
    bm = BlockManager(6, 4, list(range(6)))
    bm.attach_host(2)
    bm.add(0)
    bm.append([0], [12])          # 3 blocks, host has 2 frames
    before = state(bm)
    with pytest.raises(MemoryError):
        bm.swap_out(0)
    assert state(bm) == before
    bm.add(1)
    bm.append([1], [8])           # 2 blocks
    assert len(bm.swap_out(1)) == 2
    bm.add(2)
    bm.append([2], [12])          # 3 of the 3 free blocks; 0 left
    before = state(bm)
    with pytest.raises(MemoryError):
        bm.swap_in(1)
    assert state(bm) == before
    bm.release(2)
    assert [f for f, _ in bm.swap_in(1)] == [0, 1]
    bm.check()


def random_swap_program(seed, steps=300):
    rng = random.Random(seed)
    B = rng.choice([1, 2, 4, 16])
    bm = BlockManager(rng.randint(8, 40), B)
    bm.attach_host(rng.randint(4, 30))
    store = KVStore(2, bm.num_blocks, B, 1, 32, np.uint16)
    live, nxt, stamp = [], 0, [0]

    def write(seq, slots):
        for slot in slots:
            stamp[0] += 1
            row = np.full((1, 1, 32), stamp[0] % 65536, np.uint16)
            for layer in range(2):
                store.write(layer, [slot], row, row + 1)

    contents = {}
    done = {"out": 0, "in": 0}
    for _ in range(steps):
        op = rng.random()
        resident = [s for s in live if not bm.swapped(s)]
        try:
            if op < 0.15 or not live:
                bm.add(nxt); live.append(nxt); nxt += 1
            elif op < 0.45 and resident:
                s = rng.choice(resident)
                before = state(bm)
                try:
                    slots, pairs = bm.append([s], [rng.randint(0, 3 * B)])
                except MemoryError:
                    assert state(bm) == before
                    continue
                store.copy_blocks(pairs)
                write(s, slots)
            elif op < 0.55 and resident:
                s = rng.choice(resident)
                bm.fork(s, nxt); live.append(nxt); nxt += 1
            elif op < 0.7 and resident:
                s = rng.choice(resident)
                snap = [store.gather(layer, bm.table(s), bm.length(s)) for layer in range(2)]
                before = state(bm)
                try:
                    pairs = bm.swap_out(s)
                except MemoryError:
                    assert state(bm) == before
                    continue
                store.to_host(pairs)
                if bm.swapped(s):
                    contents[s] = snap
                    done["out"] += 1
            elif op < 0.85 and any(bm.swapped(s) for s in live):
                s = rng.choice([s for s in live if bm.swapped(s)])
                before = state(bm)
                try:
                    pairs = bm.swap_in(s)
                except MemoryError:
                    assert state(bm) == before
                    continue
                store.from_host(pairs)
                got = [store.gather(layer, bm.table(s), bm.length(s)) for layer in range(2)]
                for (k0, v0), (k1, v1) in zip(contents.pop(s), got):
                    assert np.array_equal(k0, k1) and np.array_equal(v0, v1)
                done["in"] += 1
            elif live:
                s = rng.choice(live)
                bm.release(s); live.remove(s); contents.pop(s, None)
        finally:
            bm.check()
    return done


@pytest.mark.parametrize("seed", range(12))
def test_random_programs_conserve_and_round_trip(seed):
    done = random_swap_program(seed)
    assert done["out"] >= 3 and done["in"] >= 3, done


def test_tool_pause_workload_round_trip():
    """The paused sequences read exactly their own rows after coming back, in other blocks."""
    wl = workloads.tool_pause(layers=1)
    ref = OracleReplay(wl).run()
    def pairs_of(kind, seq):
        return next(r["pairs"] for r in ref.swaps if r["kind"] == kind and r["seq"] == seq)

    out0, in0 = pairs_of("swap_out", 0), pairs_of("swap_in", 0)
    assert len(out0) == 144 and [f for f, _ in in0] == [f for _, f in out0]
    assert set(b for b, _ in out0) != set(b for _, b in in0)
    assert len(pairs_of("swap_out", 3)) == 1  # the forks share the other 62 blocks of sequence 3
    assert next(r["positions"] for r in ref.swaps if r["kind"] == "swap_out" and r["seq"] == 3) == [62]
    # the final decode's tables gather the draws each sequence wrote, wherever they live
    from synth import draws
    from synth.draws import TAG_K
    last = ref.decodes[-1]
    for s, table, n in zip(last["seq_ids"], last["tables"], last["lengths"]):
        if s in (6, 7):
            continue  # forks: their first 1000 rows were written by sequence 3
        k, _ = ref.store.gather(0, table, n)
        expect = draws.token_rows(wl.seed, TAG_K, 0, s, np.arange(n), wl.num_kv_heads, wl.head_dim, wl.dtype)
        assert np.array_equal(k, expect), s
    ref.bm.check()


def test_eager_decodes_equal_lazy_ones_where_nothing_is_reused():
    """Eager evaluation (needed once freed blocks are reused) agrees with the end-of-replay
    evaluation wherever the blocks a decode read are unchanged at the end: the last decode."""
    wl = workloads.tool_pause(layers=1)
    eager = OracleReplay(wl, eager=True).run()
    lazy = OracleReplay(wl).run()
    last = len(lazy.decodes) - 1
    np.testing.assert_array_equal(eager.attention(last, 0), lazy.attention(last, 0))
    # an empty sequence has no defined output: NaN rows in the eager record
    first = eager.attention(0, 0)
    assert np.isnan(first[5]).all() and np.isfinite(np.delete(first, 5, axis=0)).all()
