"""Prefix cache: the oracle pinned against the pages, and the library's radix
tree checked bit for bit against the oracle on random programs (CPU only).

Pins: the worked example of block-aligned truncation (100 tokens at B = 16 ->
6 shared blocks, a 4-token tail recomputed) and estimate 0.4 (footprint and
prefill work of a 4096-token prefix); brute-force longest match over every
inserted prompt; the eviction rules (only dormant leaves, oldest first, a
childless dormant parent next) checked on every eviction of random programs;
block conservation with the tree's references.
"""

import numpy as np
import pytest

from oracle.block_manager import BlockManager
from oracle.footprint import kv_bytes_per_token
from oracle.prefix_cache import PrefixCache, prefill_flops
from pagedattention_decode_amd import binding as B
from pagedattention_decode_amd.pool import PagedKVPool
from tests.prefix_programs import make_program


def test_worked_truncation_example(golden):
    s_match, bs, full, tail, usable = (int(x) for x in golden("prefix_cache.txt")["match"][0])
    bm = BlockManager(16, bs)
    pc = PrefixCache(bm)
    prompt = list(range(1000, 1000 + 7 * bs))           # 112 tokens, 7 full blocks
    bm.add("a")
    bm.append(["a"], [len(prompt)])
    assert pc.insert("a", prompt) == len(prompt)
    query = prompt[:s_match] + [-1] * 20                 # agrees on exactly s_match tokens
    m, u, blocks = pc.match(query)
    assert (m, u) == (s_match, usable)
    assert len(blocks) == full and u == full * bs and m - u == tail
    assert blocks == bm.table("a")[:full]
    assert pc.attach("b", query) == usable               # the tail is recomputed
    assert bm.table("b") == blocks and bm.length("b") == usable


def test_estimate_0_4(golden):
    g = golden("prefix_cache.txt")
    L, hkv, d, b, per_tok, S, kib, tp, mib = (int(x) for x in g["footprint"][0])
    assert kv_bytes_per_token(L, hkv, d, b) == per_tok
    assert S * per_tok == kib * 1024 and kib / 1024 / 1024 == 1.25
    assert kib / 1024 / tp == mib
    n, s, layers, dm, lin, att, tot = g["flops"][0]
    f = prefill_flops(float(n), int(s), int(layers), int(dm))
    assert abs(2 * float(n) * int(s) / 1e12 - float(lin)) < 0.05
    assert abs(4 * int(layers) * int(dm) * int(s) ** 2 / 1e12 - float(att)) < 0.05
    assert abs(f / 1e12 - float(tot)) < 0.1
    gpus, each, mfu, sustained, ms = g["ttft"][0]
    assert abs(float(mfu) * int(gpus) * float(each) - float(sustained)) < 1.0
    assert abs(f / 1e12 / float(sustained) * 1e3 - float(ms)) < 0.1


# ---------------------------------------------------------------------------
# replay of a random program on the oracle and on the library
# ---------------------------------------------------------------------------

NUM_BLOCKS, BS = 48, 4


def run_oracle(ops, order):
    bm = BlockManager(NUM_BLOCKS, BS, order)
    pc = PrefixCache(bm)
    prompts, trace = {}, []
    inserted = []  # (cached tokens) per insert, for the brute-force check
    evicted = [False]
    for op in ops:
        kind = op[0]
        if kind == "attach":
            _, s, prompt = op
            c = pc.attach(s, prompt)
            try:
                bm.append([s], [len(prompt) - c])
                ok = True
            except MemoryError:
                ok = False
            prompts[s] = prompt
            trace.append(("attach", c, ok))
        elif kind == "insert":
            s = op[1]
            toks = prompts[s][:bm.length(s)]
            c = pc.insert(s, toks)
            inserted.append(toks[:c])
            trace.append(("insert", c))
        elif kind == "release":
            trace.append(("release", pc.release(op[1])))
        elif kind == "evict":
            before = {id(n): n for n in pc.nodes()}
            dormant_leaves = [n for n in before.values() if not n.children and n.ref_count == 0]
            got = pc.evict(op[1])
            evicted[0] |= bool(got)
            trace.append(("evict", got))
            check_eviction(pc, before, dormant_leaves, got)
        else:
            m, u, blocks = pc.match(op[1])
            trace.append(("match", m, u, blocks))
            check_brute_force(op[1], m, u, inserted, exact=not evicted[0])
        bm.check()
        trace.append(("state", list(bm.free), list(bm.ref), {s: bm.table(s) for s in bm.tables},
                      {s: bm.length(s) for s in bm.lengths}))
    return trace


def check_eviction(pc, before, dormant_leaves, evicted_blocks):
    """Evicted nodes were dormant leaves when taken, oldest first; pinned nodes stay."""
    after = {id(n) for n in pc.nodes()}
    gone = [n for k, n in before.items() if k not in after]
    assert sum(len(n.blocks) for n in gone) == len(evicted_blocks)
    for n in gone:
        assert n.ref_count == 0 and not n.children
    for n in before.values():
        if n.ref_count > 0:
            assert id(n) in after
    # the first node taken is the oldest dormant leaf at the start
    if gone:
        first = min(dormant_leaves, key=lambda n: (n.last_access, n.order))
        assert evicted_blocks[:len(first.blocks)] == first.blocks


def check_brute_force(query, m, u, inserted, exact):
    """The match never exceeds the best common prefix with any inserted prompt's
    cached part; before any eviction it equals it."""
    best_full, best_tok = 0, 0
    for toks in inserted:
        k = 0
        while k < len(toks) and k < len(query) and toks[k] == query[k]:
            k += 1
        best_tok = max(best_tok, k)
        best_full = max(best_full, k // BS * BS)
    assert u % BS == 0 and u <= m and m - u < BS
    assert u <= best_full and m <= best_tok
    if exact:
        assert (m, u) == (best_tok, best_full)


def run_library(ops, order):
    pool = PagedKVPool(1, NUM_BLOCKS, BS, 1, 32, "f32", free_order=order, allocate=False)
    prompts, trace = {}, []
    for op in ops:
        kind = op[0]
        if kind == "attach":
            _, s, prompt = op
            c = pool.attach_prefix(s, prompt)
            try:
                pool.append([s], [len(prompt) - c])
                ok = True
            except B.KVOutOfBlocks:
                ok = False
            prompts[s] = prompt
            trace.append(("attach", c, ok))
        elif kind == "insert":
            s = op[1]
            trace.append(("insert", pool.prefix_insert(s, prompts[s][:pool.info(s)[0]])))
        elif kind == "release":
            before = set(pool.free_list())
            pool.release_fenced(op[1], 0)
            trace.append(("release", [b for b in pool.free_list() if b not in before]))
        elif kind == "evict":
            trace.append(("evict", pool.prefix_evict(op[1], fence=0)))
        else:
            m, u = pool.prefix_match(op[1])
            trace.append(("match", m, u))
        pool.check()
        seqs = sorted(s for s in prompts if _alive(pool, s))
        tables, lens = pool.tables(seqs, 64) if seqs else (np.zeros((0, 64), np.int32), np.zeros(0, np.int32))
        trace.append(("state", pool.free_list(), pool.refcounts(),
                      {s: [int(x) for x in tables[i] if x >= 0] for i, s in enumerate(seqs)},
                      {s: int(lens[i]) for i, s in enumerate(seqs)}))
    return trace


def _alive(pool, s):
    try:
        pool.info(s)
        return True
    except B.KVError:
        return False


def normalise(trace):
    out = []
    for item in trace:
        if item[0] == "match":
            out.append(item[:3])
        elif item[0] == "state":
            _, free, ref, tables, lens = item
            out.append(("state", [int(x) for x in free], [int(x) for x in ref],
                        {k: [int(x) for x in v] for k, v in sorted(tables.items())},
                        {k: int(v) for k, v in sorted(lens.items())}))
        elif item[0] == "release":
            out.append(("release", sorted(int(x) for x in item[1])))
        else:
            out.append(item)
    return out


@pytest.mark.parametrize("evictions", [True, False])
@pytest.mark.parametrize("seed", range(8))
def test_library_matches_oracle_on_random_programs(seed, evictions):
    ops = make_program(seed, block_size=BS, evictions=evictions)
    order = list(np.random.default_rng(seed + 100).permutation(NUM_BLOCKS))
    want = normalise(run_oracle(ops, order))
    got = normalise(run_library(ops, order))
    assert len(want) == len(got)
    for i, (w, g) in enumerate(zip(want, got)):
        assert w == g, f"step {i}: {w[0]} differs"


def test_stats_and_pinning():
    pool = PagedKVPool(1, 16, 4, 1, 32, "f32", allocate=False)
    p = list(range(10))
    assert pool.attach_prefix(1, p) == 0
    pool.append([1], [10])
    assert pool.prefix_insert(1, p) == 8
    st = pool.prefix_stats()
    assert st == {"n_nodes": 1, "n_cached_blocks": 2, "n_pinned": 1}
    assert pool.prefix_evict(16, fence=0) == []          # pinned: nothing evictable
    pool.release_fenced(1, 0)
    assert pool.prefix_stats()["n_pinned"] == 0
    assert pool.prefix_match(p + [99]) == (8, 8)          # tokens 8, 9 never filled a block
    assert pool.prefix_match(p[:6] + [99]) == (6, 4)
    assert pool.attach_prefix(2, p + [5]) == 8
    pool.release_fenced(2, 0)
    free_before = len(pool.free_list())
    evicted = pool.prefix_evict(16, fence=0)
    assert len(evicted) == 2 and len(pool.free_list()) == free_before + 2
    assert pool.prefix_stats() == {"n_nodes": 0, "n_cached_blocks": 0, "n_pinned": 0}
    pool.check()
