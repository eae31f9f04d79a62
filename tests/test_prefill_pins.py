"""Pins of the oracle's multi-query (chunked prefill / verification) attention.

The chunk attention of oracle.prefill is checked against values the pages
print (query-key pair counts, chunk ranges), against torch's fp64 causal
scaled-dot-product attention on the whole prompt (a library routine that knows
nothing of chunks or paging), against the oracle's separately pinned decode
attention (a one-row chunk), closed forms and pure-Python brute force; planted
mistakes in copies of it must each fail at least one pin.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as att
from oracle import prefill as pf
from oracle.runner import OracleReplay
from synth import draws, workloads


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_pair_counts(golden):
    rows = golden("chunk_pairs.txt")["pairs"]
    assert len(rows) == 4
    for h, c, n in rows:
        assert pf.visible_pairs(int(h), int(c)) == int(n)


def test_pair_count_closed_form():
    for h in (0, 1, 5, 16, 100):
        for c in (1, 2, 7, 16, 33):
            assert pf.visible_pairs(h, c) == c * h + c * (c + 1) // 2


def test_chunk_ranges(golden):
    g = golden("chunk_ranges.txt")
    prompt, chunk = int(g["prompt"][0][0]), int(g["chunk"][0][0])
    ranges = pf.chunk_ranges(prompt, chunk)
    assert len(ranges) == int(g["n_chunks"][0][0])
    k, first, last, ext = (int(x) for x in g["range"][0])
    assert ranges[k - 1] == (first, last)
    assert ranges[k - 1][1] + 1 == ext  # K_{<=k} holds every token up to the chunk's last
    # the ranges tile the prompt, in order, ragged last chunk included
    for S, C in ((2048, 512), (2049, 512), (5, 7), (100, 32)):
        r = pf.chunk_ranges(S, C)
        assert r[0][0] == 0 and r[-1][1] == S - 1
        assert all(b[0] == a[1] + 1 for a, b in zip(r, r[1:]))
        assert all(b - a + 1 == C for a, b in r[:-1])


# ---------------------------------------------------------------------------
# attention pins: fn(q [c, Hq, d], k [n, Hkv, d], v) -> [c, Hq, d]
# ---------------------------------------------------------------------------

def _torch_causal(q, k, v):
    """Monolithic causal attention of a whole prompt (c = n) with torch's fp64 SDPA."""
    g = q.shape[1] // k.shape[1]
    tq = torch.from_numpy(q.transpose(1, 0, 2).copy())[None]
    tk = torch.from_numpy(np.repeat(k, g, axis=1).transpose(1, 0, 2).copy())[None]
    tv = torch.from_numpy(np.repeat(v, g, axis=1).transpose(1, 0, 2).copy())[None]
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    return out[0].numpy().transpose(1, 0, 2)


def check_library_monolithic(fn):
    """No history: the chunk is the whole prompt; equals torch's causal SDPA."""
    rng = np.random.default_rng(11)
    ok = True
    for hq, hkv, d, n in ((4, 4, 8, 1), (8, 2, 16, 37), (6, 3, 32, 64)):
        q, k, v = _rand(rng, n, hq, d) * 2, _rand(rng, n, hkv, d), _rand(rng, n, hkv, d)
        ok &= np.allclose(fn(q, k, v), _torch_causal(q, k, v), rtol=0, atol=1e-12)
    return ok


def check_chunks_equal_monolithic(fn):
    """Prompt processed chunk by chunk over its history equals the monolithic result."""
    rng = np.random.default_rng(12)
    hq, hkv, d, S = 8, 2, 16, 45
    q, k, v = _rand(rng, S, hq, d) * 2, _rand(rng, S, hkv, d), _rand(rng, S, hkv, d)
    ref = _torch_causal(q, k, v)
    ok = True
    for C in (1, 7, 16, 45):
        for first, last in pf.chunk_ranges(S, C):
            got = fn(q[first:last + 1], k[:last + 1], v[:last + 1])
            ok &= np.allclose(got, ref[first:last + 1], rtol=0, atol=1e-12)
    return ok


def check_single_row_is_decode(fn):
    """A one-token chunk is a decode query over the whole context."""
    rng = np.random.default_rng(13)
    ok = True
    for n in (1, 2, 30):
        q, k, v = _rand(rng, 1, 8, 16), _rand(rng, n, 4, 16), _rand(rng, n, 4, 16)
        ok &= np.allclose(fn(q, k, v)[0], att.decode_attention(q[0], k, v), rtol=0, atol=1e-13)
    return ok


def check_identical_keys(fn):
    """Equal keys give uniform weights: row j is the mean of v_0 .. v_{h+j}."""
    rng = np.random.default_rng(14)
    hq, hkv, d, h, c = 4, 2, 8, 5, 6
    k = np.broadcast_to(_rand(rng, 1, hkv, d), (h + c, hkv, d)).copy()
    v = _rand(rng, h + c, hkv, d)
    q = _rand(rng, c, hq, d)
    out = fn(q, k, v)
    ok = True
    for j in range(c):
        mean = v[:h + j + 1].mean(axis=0)
        ok &= np.allclose(out[j], np.repeat(mean, hq // hkv, axis=0), rtol=0, atol=1e-13)
    return ok


def check_brute_force(fn):
    """Pure-Python masked softmax on a tiny chunk over a short history."""
    rng = np.random.default_rng(15)
    hq, hkv, d, h, c = 4, 2, 4, 3, 4
    q, k, v = _rand(rng, c, hq, d), _rand(rng, h + c, hkv, d), _rand(rng, h + c, hkv, d)
    out = fn(q, k, v)
    for j in range(c):
        for hh in range(hq):
            g = hh * hkv // hq
            keys = range(h + j + 1)
            s = [sum(q[j][hh][i] * k[t][g][i] for i in range(d)) / math.sqrt(d) for t in keys]
            e = [math.exp(x) for x in s]
            for i in range(d):
                val = sum(e[t] * v[t][g][i] for t in keys) / sum(e)
                if abs(val - out[j][hh][i]) > 1e-12:
                    return False
    return True


PREFILL_PINS = [check_library_monolithic, check_chunks_equal_monolithic, check_single_row_is_decode,
                check_identical_keys, check_brute_force]


@pytest.mark.parametrize("pin", PREFILL_PINS, ids=lambda f: f.__name__)
def test_prefill_pins(pin):
    assert pin(pf.chunk_attention)


def _mutants():
    """Copies of chunk_attention with one plausible mistake each."""
    def masked(rule):
        def fn(q, k, v):
            c, hq, d = q.shape
            n, hkv, _ = k.shape
            h = n - c
            out = np.empty((c, hq, d))
            for j in range(c):
                for hh in range(hq):
                    g = hh // (hq // hkv)
                    vis = np.array([rule(t, j, h) for t in range(n)])
                    if not vis.any():
                        vis[0] = True
                    s = np.where(vis, k[:, g, :] @ q[j, hh] / math.sqrt(d), -np.inf)
                    w = np.exp(s - s.max()); w /= w.sum()
                    out[j, hh] = w @ v[:, g, :]
            return out
        fn.__name__ = rule.__name__
        return fn

    def off_by_one(t, j, h):  # a query does not see its own token
        return t < h + j

    def top_left(t, j, h):  # causal mask aligned to the chunk start, history ignored
        return t <= j

    def history_hidden(t, j, h):  # only the chunk's own tokens are visible
        return h <= t <= h + j

    def no_causal(t, j, h):  # the whole chunk visible to every row
        return True

    def one_ahead(t, j, h):  # sees the next token too
        return t <= h + j + 1

    def no_scale(q, k, v):
        return pf.chunk_attention(q, k, v, scale=1.0)

    def wrong_group(q, k, v):
        hq, hkv = q.shape[1], k.shape[1]
        perm = np.array([(h % hkv) * (hq // hkv) + h // hkv for h in range(hq)])
        return pf.chunk_attention(q[:, perm], k, v)[:, np.argsort(perm)]

    return [masked(off_by_one), masked(top_left), masked(history_hidden), masked(no_causal),
            masked(one_ahead), no_scale, wrong_group]


@pytest.mark.parametrize("mutant", _mutants(), ids=lambda f: f.__name__)
def test_planted_mistakes_are_caught(mutant):
    assert not all(pin(mutant) for pin in PREFILL_PINS)


# ---------------------------------------------------------------------------
# replay: chunks through the paged pool equal the monolithic prompt
# ---------------------------------------------------------------------------

def test_replayed_chunks_equal_monolithic_prompt():
    """[KVM] Figure 8 at a small width: prompts prefilled in chunks through a shuffled
    paged pool equal torch's causal attention over the contiguous prompt."""
    wl = workloads.chunked_prompt((200, 77, 16), chunk=64)
    ref = OracleReplay(wl).run()
    assert len(ref.prefills) == 4
    # the K/V rows of a prompt, contiguous, straight from the generator
    q_rows = {s: [] for s in range(3)}
    for i, rec in enumerate(ref.prefills):
        qb = draws.bits_to_f64(ref.prefill_query_bits(i, 0), wl.dtype)
        at = 0
        for s, c in zip(rec["seq_ids"], rec["counts"]):
            q_rows[s].append(qb[at:at + c])
            at += c
    got = {s: [] for s in range(3)}
    for i, rec in enumerate(ref.prefills):
        out = ref.prefill_attention(i, 0)
        for b, s in enumerate(rec["seq_ids"]):
            got[s].append(out[b])
    for s, S in enumerate((200, 77, 16)):
        pos = np.arange(S)
        k = draws.bits_to_f64(draws.token_rows(wl.seed, draws.TAG_K, 0, s, pos, wl.num_kv_heads,
                                               wl.head_dim, wl.dtype), wl.dtype)
        v = draws.bits_to_f64(draws.token_rows(wl.seed, draws.TAG_V, 0, s, pos, wl.num_kv_heads,
                                               wl.head_dim, wl.dtype), wl.dtype)
        mono = _torch_causal(np.concatenate(q_rows[s]), k, v)
        np.testing.assert_allclose(np.concatenate(got[s]), mono, rtol=0, atol=1e-12)
    # the tables are scattered: the shuffled free list did not hand out blocks in order
    t0 = ref.prefills[-1]["tables"][0]
    assert t0 != sorted(t0)


def test_prefill_rows_match_chunk_attention():
    wl = workloads.chunked_prompt((100, 37), chunk=32)
    ref = OracleReplay(wl).run()
    full = ref.prefill_attention(1, 0)
    picks = [(0, 0), (0, 31), (1, 0), (1, 4)]
    rows = ref.prefill_rows(1, 0, picks)
    for r, (b, j) in zip(rows, picks):
        np.testing.assert_allclose(r, full[b][j], rtol=0, atol=1e-13)
    # the first rows of a chunk see no key past h + rows - 1: cutting the keys there changes nothing
    head = ref.prefill_attention(1, 0, first_rows=5)
    for b in head:
        np.testing.assert_allclose(head[b], full[b][:5], rtol=0, atol=1e-13)
