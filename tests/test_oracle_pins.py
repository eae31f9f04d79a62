"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values the
pages print (fixtures under tests/golden/, each citing its source), closed
forms, invariants, special cases that reduce to a library routine, and brute
force on tiny inputs.  ``test_planted_mistakes_are_caught`` plants plausible
mistakes in copies of the oracle's attention and checks that the attention
pins reject every one of them.
"""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import attention as att
from oracle import footprint as fp
from oracle.block_manager import BlockManager
from oracle.kv_store import KVStore
from oracle.runner import OracleReplay
from synth import draws, workloads


def _ints(vals):
    return [int(x) for x in vals]


def _order(first, n):
    rest = [b for b in range(n) if b not in first]
    return list(first) + rest


# ---------------------------------------------------------------------------
# footprint and translation facts
# ---------------------------------------------------------------------------

def test_footprints(golden):
    rows = golden("footprints.txt")
    assert rows  # fixture parsed
    for key, vals in rows.items():
        for v in vals:
            L, hkv, d, b, expect = _ints([key] + v)
            assert fp.kv_bytes_per_token(L, hkv, d, b) == expect


def test_exercise_block_bytes(golden):
    g = {k: int(v[0][0]) for k, v in golden("exercise_block_bytes.txt").items()}
    bb = fp.block_bytes(g["layers"], g["kv_heads"], g["block_size"], g["head_dim"], g["elem_bytes"])
    assert bb == g["block_bytes"]
    assert g["budget_bytes"] // bb == g["blocks"]


def test_worked_block_table(golden):
    g = golden("block_table_worked.txt")
    B = int(g["block_size"][0][0])
    first = _ints(g["free_order"][0])
    bm = BlockManager(16, B, _order(first, 16))
    bm.add("A")
    slots, pairs = bm.append(["A"], [7])
    assert pairs == []
    assert bm.table("A") == [7, 1]
    for pos, p, r in (_ints(v) for v in g["translate"]):
        assert fp.translate(pos, B, bm.table("A")) == (p, r)
        assert slots[pos] == p * B + r
    for tok, p, r, table in g["append"]:
        assert bm.length("A") == int(tok) - 1
        (slot,), _ = bm.append(["A"])
        assert slot == int(p) * B + int(r)
        assert bm.table("A") == _ints(table.split(","))
    bm.check()


def test_exercise_translation(golden):
    g = golden("exercise_translation.txt")
    B = int(g["block_size"][0][0])
    table = _ints(g["table"][0])
    for pos, p, r in (_ints(v) for v in g["translate"]):
        assert fp.translate(pos, B, table) == (p, r)
    n, waste = _ints(g["waste_at_length"][0])
    assert fp.tail_waste(n, B) == waste


def test_tail_waste_bound_brute_force():
    for B in range(1, 33):
        bm = BlockManager(64, B)
        bm.add(0)
        for n in range(0, 4 * B + 1):
            if n:
                bm.append([0])
            allocated = len(bm.table(0)) * B
            waste = allocated - n
            assert waste == fp.tail_waste(n, B) == (B - n % B) % B
            assert 0 <= waste <= B - 1
        bm.check()


def test_tail_waste_mean():
    for B in range(1, 65):
        assert fp.mean_tail_waste(B) == Fraction(B - 1, 2)
    assert float(fp.mean_tail_waste(16)) == 7.5


def test_paging_example(golden):
    g = {k: _ints(v[0]) for k, v in golden("paging_example.txt").items()}
    B = g["block_size"][0]
    bm = BlockManager(64, B)
    for s, n in enumerate(g["lengths"]):
        bm.add(s)
        bm.append([s], [n])
    alloc = [len(bm.table(s)) * B for s in range(4)]
    assert alloc == g["allocated"]
    assert sum(alloc) == g["total_allocated"][0]
    assert sum(g["lengths"]) == g["total_tokens"][0]
    assert len(g["lengths"]) * g["reservation"][0] - sum(g["lengths"]) == g["unused_reserved"][0]
    assert sum(alloc) - sum(g["lengths"]) == g["unused_paged"][0]
    # A and B share their first tokens: B forks from A at the shared prefix.
    bm = BlockManager(64, B)
    a_len, b_len, c_len, d_len = g["lengths"]
    bm.add("A")
    bm.append(["A"], [g["shared_prefix_tokens"][0]])
    bm.fork("A", "B")
    bm.append(["A", "B"], [a_len - g["shared_prefix_tokens"][0], b_len - g["shared_prefix_tokens"][0]])
    for s, n in (("C", c_len), ("D", d_len)):
        bm.add(s)
        bm.append([s], [n])
    bm.check()
    assert bm.n_allocated() * B == g["total_allocated_shared"][0]


def test_sharing_count(golden):
    g = {k: int(v[0][0]) for k, v in golden("sharing_count.txt").items()}
    B = 16
    bm = BlockManager(1024, B)
    bm.add(0)
    bm.append([0], [g["shared_blocks"] * B])
    for c in range(1, g["branches"]):
        bm.fork(0, c)
    branches = list(range(g["branches"]))
    slots, pairs = bm.append(branches, [g["private_blocks"] * B] * g["branches"])
    assert pairs == []  # the prefix ends on a block boundary: no copy needed
    bm.check()
    assert sum(len(bm.table(s)) for s in branches) == g["table_references"]
    assert bm.n_allocated() == g["physical_blocks"]
    assert bm.n_shared() == g["shared_blocks"]


def test_shared_capacity(golden):
    g = {k: int(v[0][0]) for k, v in golden("shared_capacity.txt").items()}
    per_tok = fp.kv_bytes_per_token(36, 8, 128, 2)
    assert per_tok == g["kib_per_token"] * 1024
    mib = lambda tokens: tokens * per_tok // (1024 * 1024)  # noqa: E731
    B = 16
    assert mib(fp.blocks_needed(g["short_tokens"], B) * B) == g["short_mib"]
    assert mib(fp.blocks_needed(g["long_tokens"], B) * B) == g["long_mib"]
    assert mib(g["prefix_tokens"]) == g["prefix_mib"]
    private = g["long_tokens"] - g["prefix_tokens"]
    bm = BlockManager(4096, B)
    bm.add(0)
    bm.append([0], [g["prefix_tokens"]])
    for c in range(1, 16):
        bm.fork(0, c)
    bm.append(list(range(16)), [private] * 16)
    bm.check()
    assert mib(bm.n_allocated() * B) == g["shared16_mib"]
    assert 16 * g["long_mib"] == g["independent16_mib"]
    assert g["budget_mib"] // g["short_mib"] == g["fit_short"]
    assert g["budget_mib"] // g["long_mib"] == g["fit_long"]
    assert (g["budget_mib"] - g["prefix_mib"]) // g["short_mib"] == g["fit_long_shared"]


def test_fork_figure(golden):
    g = golden("fork_figure.txt")
    B = int(g["block_size"][0][0])
    shared = dict(tuple(map(int, x.split(":"))) for x in g["shared"][0])
    a2 = int(g["a_logical2"][0][0])
    new = int(g["b_new_block"][0][0])
    bm = BlockManager(16, B, _order([shared[0], shared[1], a2, new], 16))
    bm.add("A")
    bm.append(["A"], [2 * B + 1])  # logical block 2 partly filled
    bm.fork("A", "B")
    assert bm.table("B")[:2] == [shared[0], shared[1]]
    assert bm.ref[shared[0]] == bm.ref[shared[1]] == 2
    (slot,), pairs = bm.append(["B"])
    assert pairs == [(a2, new)]
    assert bm.table("B") == [shared[0], shared[1], new]
    assert bm.table("A") == [shared[0], shared[1], a2]
    assert slot == new * B + 1
    # A is now the only holder of its block: it writes in place, no copy.
    (slot,), pairs = bm.append(["A"])
    assert pairs == [] and slot == a2 * B + 1
    bm.check()


def test_pool_70b(golden):
    g = {k: int(v[0][0]) for k, v in golden("pool_70b.txt").items()}
    assert fp.kv_bytes_per_token(80, 1, 128, 2) == g["kib_per_token"] * 1024
    assert fp.block_bytes(80, 1, 16, 128, 2) == g["block16_kib"] * 1024
    assert fp.block_bytes(80, 1, 64, 128, 2) == g["block64_kib"] * 1024
    assert g["pool_kib"] // g["block16_kib"] == g["pool_blocks16"]
    assert g["pool_blocks16"] * 16 == g["pool_tokens16"]
    assert fp.mean_tail_waste(16) * 2 == g["mean_waste16_x2"]
    assert fp.mean_tail_waste(64) * 2 == g["mean_waste64_x2"]
    assert g["sequences"] * fp.mean_tail_waste(16) * g["kib_per_token"] == g["waste16_kib"]
    assert g["sequences"] * fp.mean_tail_waste(64) * g["kib_per_token"] == g["waste64_kib"]
    assert round(100 * 100 * g["waste16_kib"] / 1024 / g["pool_mib"]) == g["ratio16_pct_x100"]
    assert round(100 * 100 * g["waste64_kib"] / 1024 / g["pool_mib"]) == g["ratio64_pct_x100"]


# ---------------------------------------------------------------------------
# block manager invariants and failure handling
# ---------------------------------------------------------------------------

def _snapshot(bm):
    return (list(bm.free), list(bm.ref), {s: list(t) for s, t in bm.tables.items()}, dict(bm.lengths))


def test_conservation_random_programs():
    rng = np.random.default_rng(7)
    for trial in range(30):
        B = int(rng.choice([1, 2, 4, 16]))
        N = int(rng.integers(4, 40))
        bm = BlockManager(N, B, rng.permutation(N))
        live, next_id = [], 0
        for _ in range(200):
            r = rng.random()
            if r < 0.15 or not live:
                bm.add(next_id)
                live.append(next_id)
                next_id += 1
            elif r < 0.3:
                bm.fork(int(rng.choice(live)), next_id)
                live.append(next_id)
                next_id += 1
            elif r < 0.45:
                s = int(rng.choice(live))
                bm.release(s)
                live.remove(s)
            else:
                k = int(rng.integers(1, len(live) + 1))
                seqs = [int(x) for x in rng.choice(live, size=k, replace=False)]
                counts = [int(x) for x in rng.integers(0, 3 * B + 1, size=k)]
                before = _snapshot(bm)
                try:
                    slots, pairs = bm.append(seqs, counts)
                except MemoryError:
                    assert _snapshot(bm) == before
                    continue
                assert len(slots) == sum(counts)
                # every slot lies in a block now owned by its sequence
                at = 0
                for s, c in zip(seqs, counts):
                    for slot in slots[at:at + c]:
                        assert slot // B in bm.tables[s]
                    at += c
                for src, dst in pairs:
                    assert bm.ref[dst] == 1
            bm.check()


def test_append_oom_rolls_back_everything():
    bm = BlockManager(5, 4, [4, 3, 2, 1, 0])
    bm.add(0)
    bm.add(1)
    bm.append([0], [6])  # blocks 4, 3
    bm.fork(0, 2)        # shares 4 and 3 (3 partly filled)
    before = _snapshot(bm)
    # seq 2 copies block 3 (1 block), seq 1 needs 3 blocks: 4 > 3 free
    with pytest.raises(MemoryError):
        bm.append([2, 1], [1, 12])
    assert _snapshot(bm) == before
    bm.check()
    # the same batch without the overflow succeeds and the copy is recorded
    slots, pairs = bm.append([2, 1], [1, 8])
    assert pairs == [(3, 2)]
    bm.check()


def test_invalid_operations():
    bm = BlockManager(4, 2)
    bm.add(0)
    with pytest.raises(ValueError):
        bm.add(0)
    with pytest.raises(ValueError):
        bm.fork(5, 6)
    with pytest.raises(ValueError):
        bm.append([9])
    with pytest.raises(ValueError):
        bm.release(9)
    with pytest.raises(ValueError):
        BlockManager(4, 2, [0, 1, 1, 2])


def test_release_returns_blocks_fifo():
    bm = BlockManager(6, 2, [5, 4, 3, 2, 1, 0])
    bm.add("a")
    bm.append(["a"], [5])  # 5, 4, 3
    bm.fork("a", "b")
    assert bm.release("a") == []  # still held by b
    assert bm.release("b") == [5, 4, 3]
    assert list(bm.free) == [2, 1, 0, 5, 4, 3]
    bm.check()


# ---------------------------------------------------------------------------
# attention: closed forms, library cross-checks, brute force, invariants
# ---------------------------------------------------------------------------

def _rand(rng, *shape):
    return rng.standard_normal(shape)


def check_two_token_closed_form(fn):
    """n = 2 keys 0 and a*e0, query c*e0: w1 = 1/(1 + exp(-a c / sqrt d))."""
    d, a, c = 16, 1.7, -2.3
    q = np.zeros((1, d)); q[0, 0] = c
    k = np.zeros((2, 1, d)); k[1, 0, 0] = a
    rng = np.random.default_rng(3)
    v = _rand(rng, 2, 1, d)
    w1 = 1.0 / (1.0 + math.exp(-a * c / math.sqrt(d)))
    expect = (1 - w1) * v[0, 0] + w1 * v[1, 0]
    return np.allclose(fn(q, k, v), expect[None], rtol=0, atol=1e-13)


def check_gqa_mapping(fn):
    """KV head g holds the constant value g in every V row: out_h = h // G."""
    rng = np.random.default_rng(4)
    hq, hkv, d, n = 12, 4, 8, 9
    q = _rand(rng, hq, d)
    k = _rand(rng, n, hkv, d)
    v = np.broadcast_to(np.arange(hkv, dtype=np.float64)[None, :, None], (n, hkv, d)).copy()
    out = fn(q, k, v)
    expect = (np.arange(hq) // (hq // hkv)).astype(np.float64)[:, None] * np.ones((1, d))
    return np.allclose(out, expect, rtol=0, atol=1e-12)


def check_library(fn):
    """Equals torch's fp64 scaled_dot_product_attention with K/V repeated per group."""
    rng = np.random.default_rng(5)
    ok = True
    for hq, hkv, d, n in ((4, 4, 8, 1), (8, 2, 16, 37), (6, 3, 32, 100), (4, 1, 64, 9)):
        q = _rand(rng, hq, d) * 2
        k = _rand(rng, n, hkv, d)
        v = _rand(rng, n, hkv, d)
        g = hq // hkv
        tq = torch.from_numpy(q)[None, :, None, :]
        tk = torch.from_numpy(np.repeat(k, g, axis=1).transpose(1, 0, 2).copy())[None]
        tv = torch.from_numpy(np.repeat(v, g, axis=1).transpose(1, 0, 2).copy())[None]
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[0, :, 0, :].numpy()
        ok &= np.allclose(fn(q, k, v), ref, rtol=0, atol=1e-12)
    return ok


def check_special_cases(fn):
    rng = np.random.default_rng(6)
    hq, hkv, d = 4, 2, 16
    ok = True
    # n = 1: the output is v_0 exactly
    q = _rand(rng, hq, d) * 5
    k = _rand(rng, 1, hkv, d)
    v = _rand(rng, 1, hkv, d)
    ok &= np.array_equal(fn(q, k, v), np.repeat(v[0], hq // hkv, axis=0))
    # all keys equal: uniform weights, the output is the mean of v
    n = 11
    k = np.broadcast_to(_rand(rng, 1, hkv, d), (n, hkv, d)).copy()
    v = _rand(rng, n, hkv, d)
    ok &= np.allclose(fn(q, k, v), np.repeat(v.mean(axis=0), hq // hkv, axis=0), atol=1e-13)
    # q = 0: uniform weights as well
    k = _rand(rng, n, hkv, d)
    ok &= np.allclose(fn(np.zeros((hq, d)), k, v), np.repeat(v.mean(axis=0), hq // hkv, axis=0),
                      atol=1e-13)
    return ok


def check_brute_force(fn):
    """Pure-Python evaluation of sum_t e^{s_t} v_t / sum_t e^{s_t} on tiny inputs."""
    rng = np.random.default_rng(8)
    hq, hkv, d, n = 4, 2, 4, 7
    q = _rand(rng, hq, d)
    k = _rand(rng, n, hkv, d)
    v = _rand(rng, n, hkv, d)
    out = fn(q, k, v)
    for h in range(hq):
        g = h * hkv // hq
        s = [sum(q[h][i] * k[t][g][i] for i in range(d)) / math.sqrt(d) for t in range(n)]
        e = [math.exp(x) for x in s]
        for i in range(d):
            val = sum(e[t] * v[t][g][i] for t in range(n)) / sum(e)
            if abs(val - out[h][i]) > 1e-12:
                return False
    return True


ATTENTION_PINS = [check_two_token_closed_form, check_gqa_mapping, check_library,
                  check_special_cases, check_brute_force]


@pytest.mark.parametrize("pin", ATTENTION_PINS, ids=lambda f: f.__name__)
def test_attention_pins(pin):
    assert pin(att.decode_attention)


@pytest.mark.parametrize("pin", ATTENTION_PINS, ids=lambda f: f.__name__)
def test_split_k_pins(pin):
    for part in (1, 3, 16):
        assert pin(lambda q, k, v, p=part: att.split_k_attention(q, k, v, p))


def test_split_k_equals_single_pass():
    rng = np.random.default_rng(9)
    q = _rand(rng, 8, 64) * 3
    k = _rand(rng, 1000, 2, 64)
    v = _rand(rng, 1000, 2, 64)
    ref = att.decode_attention(q, k, v)
    for part in (1, 7, 16, 512, 999, 1000, 4096):
        np.testing.assert_allclose(att.split_k_attention(q, k, v, part), ref, rtol=0, atol=1e-13)


def test_merge_single_partition_is_identity():
    rng = np.random.default_rng(10)
    q, k, v = _rand(rng, 4, 8), _rand(rng, 5, 2, 8), _rand(rng, 5, 2, 8)
    m, l, o = att.partition_stats(q, k, v)
    m2, l2, o2 = att.merge_partitions([(m, l, o)])
    assert np.array_equal(m, m2) and np.array_equal(l, l2) and np.array_equal(o, o2)


def test_merge_closed_form():
    """Two partitions with one token each: the merged weights are a logistic function."""
    m = np.array([0.5]); o1 = np.array([[2.0]]); o2 = np.array([[-1.0]])
    parts = [(m, np.array([1.0]), o1), (np.array([1.75]), np.array([1.0]), o2)]
    mm, l, o = att.merge_partitions(parts)
    w2 = 1 / (1 + math.exp(0.5 - 1.75))
    assert mm[0] == 1.75
    assert abs(o[0, 0] / l[0] - ((1 - w2) * 2.0 + w2 * -1.0)) < 1e-15


def _mutants():
    """Copies of decode_attention with one plausible mistake each."""
    def no_scale(q, k, v):
        return att.decode_attention(q, k, v, scale=1.0)

    def wrong_group(q, k, v):
        hq, hkv = q.shape[0], k.shape[1]
        out = np.empty_like(q)
        for h in range(hq):
            g = h % hkv
            s = k[:, g, :] @ q[h] / math.sqrt(q.shape[1])
            w = np.exp(s - s.max()); w /= w.sum()
            out[h] = w @ v[:, g, :]
        return out

    def sign_flip(q, k, v):
        return att.decode_attention(-q, k, v)

    def transposed_kv(q, k, v):
        return att.decode_attention(q, v, k)

    def dropped_last_token(q, k, v):
        if k.shape[0] == 1:
            return att.decode_attention(q, k, v)
        return att.decode_attention(q, k[:-1], v[:-1])

    def no_normalisation(q, k, v):
        _, l, o = att.partition_stats(q, k, v)
        return o

    def off_by_one_position(q, k, v):
        return att.decode_attention(q, np.roll(k, 1, axis=0), v)

    return [no_scale, wrong_group, sign_flip, transposed_kv, dropped_last_token,
            no_normalisation, off_by_one_position]


@pytest.mark.parametrize("mutant", _mutants(), ids=lambda f: f.__name__)
def test_planted_mistakes_are_caught(mutant):
    assert not all(pin(mutant) for pin in ATTENTION_PINS)


# ---------------------------------------------------------------------------
# paged gather: sentinels, permutation invariance, forks
# ---------------------------------------------------------------------------

def _sentinel_rows(seq, positions, hkv, d):
    rows = np.empty((len(positions), hkv, d), dtype=np.float32)
    for i, t in enumerate(positions):
        rows[i] = seq * 1000 + t
    return rows.view(np.uint32)


def test_block_size_two_sentinels():
    """Block size 2, lengths 1..5 grown interleaved; every gathered row is its own sentinel."""
    B, hkv, d = 2, 1, 4
    bm = BlockManager(32, B, np.random.default_rng(11).permutation(32))
    store = KVStore(1, 32, B, hkv, d, np.uint32)
    targets = [1, 2, 3, 4, 5]
    for s in range(5):
        bm.add(s)
    lens = [0] * 5
    while any(l < t for l, t in zip(lens, targets)):
        seqs = [s for s in range(5) if lens[s] < targets[s]]
        slots, pairs = bm.append(seqs)
        assert pairs == []
        for s, slot in zip(seqs, slots):
            rows = _sentinel_rows(s, [lens[s]], hkv, d)
            store.write(0, [slot], rows, rows)
            lens[s] += 1
        bm.check()
    for s in range(5):
        k, v = store.gather(0, bm.table(s), targets[s])
        got = draws.bits_to_f64(k, draws.F32)[:, 0, 0]
        assert list(got) == [s * 1000 + t for t in range(targets[s])]


def test_permutation_invariance():
    wl = workloads.tiny_fp32()
    a = OracleReplay(wl, free_order=draws.free_order(1, 16)).run()
    b = OracleReplay(wl, free_order=draws.free_order(99, 16)).run()
    assert a.decodes[0]["tables"] != b.decodes[0]["tables"]
    assert np.array_equal(a.attention(0, 0), b.attention(0, 0))


def test_tiny_workload_replay():
    wl = workloads.tiny_fp32()
    r = OracleReplay(wl).run()
    assert r.decodes[0]["lengths"] == [5, 7, 9]
    assert [len(t) for t in r.decodes[0]["tables"]] == [2, 2, 3]
    assert r.bm.n_allocated() == 7
    r.bm.check()
    out = r.attention(0, 0)
    assert out.shape == (3, 4, 64) and np.isfinite(out).all()


def test_forks_share_then_isolate():
    wl = workloads.Workload("fork", 12, draws.BF16, 2, 8, 2, 32, 4, 64,
                            [("add", 0), ("append", (0,), (10,)), ("fork", 0, 1), ("decode", (0, 1)),
                             ("append", (1,), (3,)), ("decode", (0, 1))])
    r = OracleReplay(wl)
    r.run(wl.ops[:4])
    # identical tables before divergence -> identical outputs for the same query
    for layer in range(2):
        q = draws.bits_to_f64(r.query_bits(0, layer), wl.dtype)
        out = r.attention(0, layer)
        kb, vb = r.store.gather(layer, r.decodes[0]["tables"][0], 10)
        from oracle.attention import decode_attention
        assert np.array_equal(decode_attention(q[1], draws.bits_to_f64(kb, wl.dtype),
                                               draws.bits_to_f64(vb, wl.dtype)), out[1])
        assert r.decodes[0]["tables"][0] == r.decodes[0]["tables"][1]
    parent_blocks = {(l, p): (r.store.block("k", l, p).copy(), r.store.block("v", l, p).copy())
                     for l in range(2) for p in r.bm.table(0)}
    r.run(wl.ops[4:])
    _, _, slots, pairs = r.appends[-1]
    assert len(pairs) == 1 and pairs[0][0] == r.bm.table(0)[-1]
    # the parent's blocks are bitwise untouched, the child's rows are its own
    for (l, p), (kb, vb) in parent_blocks.items():
        assert np.array_equal(r.store.block("k", l, p), kb)
        assert np.array_equal(r.store.block("v", l, p), vb)
    assert r.bm.table(1)[2] == pairs[0][1]  # logical block 2 was copied; block 3 is new
    for l in range(2):
        ck, _ = r.store.gather(l, r.bm.table(1), 13)
        pk, _ = r.store.gather(l, r.bm.table(0), 10)
        assert np.array_equal(ck[:10], pk)  # the copied prefix matches the parent
        expect = draws.token_rows(wl.seed, draws.TAG_K, l, 1, np.arange(10, 13), 2, 32, wl.dtype)
        assert np.array_equal(ck[10:], expect)
    r.bm.check()


def test_bf16_rounding_is_nearest_even():
    """Input rounding pin: hand-checked bf16 encodings (ties go to even)."""
    x = np.array([1.0, -2.0, 1.00390625, 1.01171875, 3.140625, 1e-3], dtype=np.float32)
    bits = draws.f32_to_bf16_bits(x)
    # 1 + 2^-8 is a tie between 1.0 and 1 + 2^-7: even mantissa (1.0) wins;
    # 1 + 3*2^-8 is a tie between 1 + 2^-7 and 1 + 2^-6: even (1 + 2^-6) wins.
    assert list(bits[:5]) == [0x3F80, 0xC000, 0x3F80, 0x3F82, 0x4049]
    assert abs(draws.bits_to_f64(bits[5:], draws.BF16)[0] - 1e-3) < 2 ** -17
