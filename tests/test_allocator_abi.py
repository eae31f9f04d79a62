"""CPU tests of the C ABI: the library loads and exports every declared symbol,
and its host block manager agrees bit for bit with the oracle's block manager
(slot mappings, copy-on-write pairs, block tables, free-list order and
reference counts) on the benchmark workloads and on random programs,
including pool exhaustion (all-or-nothing batches) and deferred release.
No device work is done here: pools are created over NULL buffers.
"""

import os
import re

import numpy as np
import pytest

from oracle.block_manager import BlockManager
from pagedattention_decode_amd import binding as B
from pagedattention_decode_amd.pool import PagedKVPool
from synth import draws, workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "pagedkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][A-Za-z0-9_ \*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert "kv_pool_create" in names and "paged_attention_decode" in names
    assert "reshape_and_cache" in names and "copy_blocks" in names
    lib = B.lib()
    for n in names:
        assert hasattr(lib, n), f"{n} is declared but not exported"
    assert set(names) == set(B.SIGNATURES), "binding and header disagree"


def host_pool(wl_or_args, free_order=None):
    if isinstance(wl_or_args, workloads.Workload):
        wl = wl_or_args
        args = (wl.num_layers, wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim, wl.dtype)
    else:
        args = wl_or_args
    return PagedKVPool(*args, free_order=free_order, allocate=False)


def assert_same_state(pool: PagedKVPool, bm: BlockManager):
    assert list(pool.free_list()) == list(bm.free)
    assert list(pool.refcounts()) == bm.ref
    for s, t in bm.tables.items():
        length, nb = pool.info(s)
        assert length == bm.lengths[s] and nb == len(t)
        if t:
            tab, lens = pool.tables([s], len(t))
            assert list(tab[0]) == t and lens[0] == bm.lengths[s]
    st = pool.stats()
    assert st["n_free"] == bm.n_free() and st["n_allocated"] == bm.n_allocated()
    assert st["n_shared"] == bm.n_shared() and st["n_seqs"] == len(bm.tables)
    pool.check()
    bm.check()


def replay_both(wl):
    order = draws.free_order(wl.seed, wl.num_blocks)
    pool = host_pool(wl, order)
    bm = BlockManager(wl.num_blocks, wl.block_size, order)
    n_checked = 0
    for op in wl.ops:
        if op[0] == "add":
            pool.add(op[1]); bm.add(op[1])
        elif op[0] == "fork":
            pool.fork(op[1], op[2]); bm.fork(op[1], op[2])
        elif op[0] == "append":
            slots, pairs = pool.append(op[1], op[2])
            r_slots, r_pairs = bm.append(op[1], op[2])
            assert np.array_equal(slots, np.asarray(r_slots, np.int64))
            assert [tuple(p) for p in pairs.tolist()] == r_pairs
            n_checked += len(slots)
        elif op[0] == "decode":
            seqs = list(op[1])
            mb = max(len(bm.tables[s]) for s in seqs)
            tab, lens = pool.tables(seqs, mb + 1)
            for i, s in enumerate(seqs):
                t = bm.tables[s]
                assert list(tab[i, :len(t)]) == t and (tab[i, len(t):] == -1).all()
                assert lens[i] == bm.lengths[s]
    assert_same_state(pool, bm)
    pool.close()
    return bm, n_checked


@pytest.mark.parametrize("name, tokens", [("tiny_fp32", 21), ("qwen3_8b_37x2304", 37 * 2304),
                                          ("shared_prefix_16x8448", 6144 + 16 * 2304),
                                          ("gqa70b_12x131072", 12 * 131072)])
def test_workload_allocator_bit_exact(name, tokens):
    wl = workloads.get_workload(name)
    bm, n = replay_both(wl)
    assert n == tokens


def test_agentic_fork_allocator_bit_exact():
    wl = workloads.agentic_fork(steps=40, layers=36)
    bm, n = replay_both(wl)
    # 4 roots x 2049 shared blocks; at the first divergent append branches 0-14
    # of each root copy the partly filled last block and branch 15 writes in place
    assert bm.n_shared() == 4 * 2048
    lens = {s: bm.lengths[s] for s in range(64)}
    assert set(lens.values()) == {32769 + 40}


def test_agentic_fork_copy_count():
    wl = workloads.agentic_fork(steps=1, layers=1)
    order = draws.free_order(wl.seed, wl.num_blocks)
    pool = host_pool(wl, order)
    for op in wl.ops:
        if op[0] == "add":
            pool.add(op[1])
        elif op[0] == "fork":
            pool.fork(op[1], op[2])
        elif op[0] == "append":
            slots, pairs = pool.append(op[1], op[2])
    # the last append is the first divergent step: 15 copies per root
    assert len(pairs) == 60
    pool.check()


def random_program_check(seed):
    rng = np.random.default_rng(seed)
    Bs = int(rng.choice([1, 2, 4, 16]))
    N = int(rng.integers(4, 48))
    order = rng.permutation(N).astype(np.int32)
    pool = host_pool((1, N, Bs, 1, 32, "f32"), order)
    bm = BlockManager(N, Bs, order)
    live, nxt = [], 0
    for _ in range(150):
        r = rng.random()
        if r < 0.15 or not live:
            pool.add(nxt); bm.add(nxt); live.append(nxt); nxt += 1
        elif r < 0.3:
            p = int(rng.choice(live))
            pool.fork(p, nxt); bm.fork(p, nxt); live.append(nxt); nxt += 1
        elif r < 0.42:
            s = int(rng.choice(live))
            pool.release_fenced(s, 0); bm.release(s); live.remove(s)
        else:
            k = int(rng.integers(1, len(live) + 1))
            seqs = [int(x) for x in rng.choice(live, size=k, replace=bool(rng.random() < 0.2))]
            counts = [int(x) for x in rng.integers(0, 3 * Bs + 1, size=k)]
            try:
                r_slots, r_pairs = bm.append(seqs, counts)
                ok = True
            except MemoryError:
                ok = False
            if ok:
                slots, pairs = pool.append(seqs, counts)
                assert np.array_equal(slots, np.asarray(r_slots, np.int64))
                assert [tuple(p) for p in pairs.tolist()] == r_pairs
            else:
                with pytest.raises(B.KVOutOfBlocks):
                    pool.append(seqs, counts)
        assert_same_state(pool, bm)
    pool.close()


@pytest.mark.parametrize("seed", range(12))
def test_random_programs_bit_exact(seed):
    random_program_check(seed)


def test_oom_leaves_state_unchanged():
    pool = host_pool((1, 5, 4, 1, 32, "f32"), [4, 3, 2, 1, 0])
    pool.add(0); pool.add(1)
    pool.append([0], [6])
    pool.fork(0, 2)
    before = (list(pool.free_list()), list(pool.refcounts()), pool.tables([0, 1, 2], 8))
    with pytest.raises(B.KVOutOfBlocks):
        pool.append([2, 1], [1, 12])
    after = (list(pool.free_list()), list(pool.refcounts()), pool.tables([0, 1, 2], 8))
    assert before[0] == after[0] and before[1] == after[1]
    assert all(np.array_equal(a, b) for a, b in zip(before[2], after[2]))
    pool.check()
    slots, pairs = pool.append([2, 1], [1, 8])
    assert pairs.tolist() == [[3, 2]]
    pool.check()


def test_invalid_calls_are_rejected_without_change():
    pool = host_pool((1, 8, 4, 1, 32, "f32"))
    pool.add(1)
    for fn in (lambda: pool.add(1), lambda: pool.fork(7, 8), lambda: pool.fork(1, 1),
               lambda: pool.append([9]), lambda: pool.append([1], [-1]), lambda: pool.release_fenced(5, 0),
               lambda: pool.tables([1, 4], 2)):
        with pytest.raises(B.KVError) as e:
            fn()
        assert e.value.status == B.KV_ERR_INVALID
        assert B.kv_last_error()
    pool.append([1], [9])  # 3 blocks
    with pytest.raises(B.KVError):
        pool.tables([1], 2)  # table longer than max_blocks
    pool.check()
    cfg = B.make_config(1, 4, 4, 1, 33, B.KV_F32)
    with pytest.raises(B.KVError):
        B.kv_pool_required_bytes(cfg)
    with pytest.raises(B.KVError):
        PagedKVPool(1, 4, 4, 1, 32, "f32", free_order=[0, 1, 1, 2], allocate=False)


def test_deferred_release_waits_for_fence():
    """Released blocks are not reused until their fence is retired."""
    pool = host_pool((1, 4, 2, 1, 32, "f32"), [0, 1, 2, 3])
    a = 5
    pool.add(a)
    pool.append([a], [4])  # blocks 0, 1
    pool.add(1000)
    pool.release_fenced(a, 7)
    st = pool.stats()
    assert st["n_pending"] == 2 and st["n_free"] == 2
    pool.check()
    pool.append([1000], [4])  # blocks 2, 3; 0 and 1 are still in flight
    with pytest.raises(B.KVOutOfBlocks):
        pool.append([1000], [1])
    pool.retire(6)
    assert pool.stats()["n_pending"] == 2
    pool.retire(7)
    assert pool.stats()["n_pending"] == 0
    assert list(pool.free_list()) == [0, 1]
    slots, _ = pool.append([1000], [1])
    assert slots[0] == 0 * 2 + 0
    pool.check()


def test_release_order_and_shared_blocks():
    pool = host_pool((1, 6, 2, 1, 32, "f32"), [5, 4, 3, 2, 1, 0])
    pool.add(0)
    pool.append([0], [5])  # 5, 4, 3
    pool.fork(0, 1)
    pool.release_fenced(0, 0)
    assert list(pool.refcounts()[[5, 4, 3]]) == [1, 1, 1]
    pool.release_fenced(1, 0)
    assert list(pool.free_list()) == [2, 1, 0, 5, 4, 3]
    pool.check()


def test_empty_batches_and_zero_counts():
    pool = host_pool((1, 4, 4, 1, 32, "f32"))
    slots, pairs = pool.append([], [])
    assert slots.size == 0 and pairs.size == 0
    pool.add(3)
    slots, pairs = pool.append([3], [0])
    assert slots.size == 0
    assert pool.info(3) == (0, 0)
    pool.check()


def test_quantised_pool_sizes_and_shape_limits():
    """[INF] §8.4.2 budget: per 32 values, 32 (q8_0) or 16 (q4_0) code bytes plus a
    2-byte scale, so a tile of 16 slots x d dims takes 16 d bits/8 + d bytes."""
    from oracle import quant as qt

    for fmt, code in (("q8_0", B.KV_Q8_0), ("q4_0", B.KV_Q4_0)):
        for d in (64, 128, 256):
            cfg = B.make_config(3, 10, 16, 4, d, code)
            kb, vb = B.kv_pool_required_bytes(cfg)
            values = 3 * 10 * 4 * 16 * d
            assert kb == vb == values // 32 * qt.group_bytes(fmt)
        for bad in (B.make_config(1, 4, 8, 2, 128, code), B.make_config(1, 4, 16, 2, 96, code)):
            with pytest.raises(B.KVError) as e:
                B.kv_pool_required_bytes(bad)
            assert e.value.status == B.KV_ERR_UNSUPPORTED


# -- groups for the read-once decode over shared prefixes ----------------------

def brute_plan(tables, lengths, B_):
    """Maximal runs of consecutive sequences sharing >= 1 completely filled leading block
    with the run's first member; shared = the fewest such blocks over the run's members."""
    def common(a, b):
        lim = min(lengths[a], lengths[b]) // B_
        j = 0
        while j < lim and tables[a][j] == tables[b][j]:
            j += 1
        return j
    gs, sb, i, n = [], [], 0, len(tables)
    while i < n:
        k, shared = i + 1, None
        while k < n and common(i, k) >= 1:
            shared = common(i, k) if shared is None else min(shared, common(i, k))
            k += 1
        gs.append(i)
        sb.append(shared or 0)
        i = k
    return gs + [n], sb


def plan_of(pool, seqs):
    tables, lens = pool.tables(seqs, max(1, max(pool.info(s)[1] for s in seqs)))
    return [list(t) for t in tables], [int(x) for x in lens]


def test_shared_prefix_plan_on_workloads():
    wl = workloads.shared_prefix()
    pool = host_pool(wl, draws.free_order(wl.seed, wl.num_blocks))
    seqs = None
    for op in wl.ops:
        if op[0] == "add":
            pool.add(op[1])
        elif op[0] == "fork":
            pool.fork(op[1], op[2])
        elif op[0] == "append":
            pool.append(op[1], op[2])
        elif op[0] == "decode":
            seqs = list(op[1])
    gs, sb = pool.shared_prefix_plan(seqs)
    assert list(gs) == [0, 16] and list(sb) == [384]
    # the members in another order are still one run
    gs, sb = pool.shared_prefix_plan(seqs[:5] + [seqs[-1]] + seqs[5:-1])
    assert list(gs) == [0, 16] and list(sb) == [384]
    tables, lens = plan_of(pool, seqs)
    assert brute_plan(tables, lens, 16) == ([0, 16], [384])


def test_shared_prefix_plan_random_forks():
    rng = np.random.default_rng(7)
    for trial in range(30):
        pool = host_pool((1, 400, 4, 1, 32, "f32"))
        live, nxt = [], 0
        for _ in range(int(rng.integers(1, 12))):
            if live and rng.random() < 0.5:
                src = int(rng.choice(live))
                pool.fork(src, nxt)
            else:
                pool.add(nxt)
            live.append(nxt)
            nxt += 1
            counts = [int(rng.integers(0, 9)) for _ in live]
            pool.append(live, counts)
        order = list(rng.permutation(live)) if trial % 2 else sorted(live, key=lambda s: pool.info(s)[1])
        gs, sb = pool.shared_prefix_plan(order)
        tables, lens = plan_of(pool, order)
        assert (list(gs), list(sb)) == brute_plan(tables, lens, 4), trial
    assert list(pool.shared_prefix_plan([])[0]) == [0]
    with pytest.raises(B.KVError):
        pool.shared_prefix_plan([10 ** 6])


def test_pool_config_round_trip_and_host_tensors_refused():
    """kv_pool_get_config returns the creation config; the binding refuses device
    arguments that are not GPU tensors before calling the library."""
    import torch

    cfg = B.make_config(3, 40, 8, 2, 64, B.KV_BF16)
    pool = B.kv_pool_create(cfg, 0, 0)
    try:
        got = B.kv_pool_get_config(pool)
        assert [getattr(got, f) for f, _ in got._fields_] == [3, 40, 8, 2, 64, B.KV_BF16]
        rows = torch.zeros((2, 2, 64), dtype=torch.bfloat16)
        with pytest.raises(B.KVArgumentError) as e:
            B.reshape_and_cache(pool, 0, rows, rows, torch.zeros(2, dtype=torch.int64))
        assert "GPU" in str(e.value) and isinstance(e.value, ValueError) and e.value.status == B.KV_ERR_INVALID
    finally:
        B.kv_pool_destroy(pool)
