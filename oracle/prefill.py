"""Multi-query attention over paged history in float64 (test infrastructure; see oracle/__init__).

Chunked prefill ([KVM] chunked prefill mechanism, Figure 8 and the equations
around it): a prompt of S tokens is cut into K = ceil(S / C) consecutive
chunks, chunk k covering positions (k-1)C .. min(kC, S) - 1.  At iteration k
the queries Q_k of the chunk's tokens attend the concatenation of the cached
keys/values of chunks 1..k-1 and the chunk's own K_k, V_k:

    O_k = softmax(Q_k K_{<=k}^T / sqrt(d) + M_k) V_{<=k}

where the mask M_k lets every query see the whole history and, inside the
chunk, only tokens at or before its own position (lower-triangular causal).
Speculative verification ([INF] section 8.5.1: the target model scores all
draft positions of a request in one pass; section 8.5.2: checking 5 positions
reads the same KV as one decode step; section 8.6.3 verifies 8 positions per
request) is the same operation with a short chunk.

Reading taken here (the pages leave the order open): the chunk's own K/V rows
are written into the paged pool first, so the pool holds positions
0 .. h + c - 1 (h = history length, c = chunk length) and the mask alone
decides what each query sees: the query at chunk row j sits at position h + j
and sees cached positions t <= h + j.

[INF] section 8.2.3 counts the (query, key) pairs of one chunk:
N_pair = (h+1) + (h+2) + ... + (h+c) = c h + c(c+1)/2; :func:`visible_pairs`
counts the mask used below, so the printed values pin the mask.
"""

from __future__ import annotations

import numpy as np


def chunk_ranges(prompt_tokens, chunk_tokens):
    """[(first, last)] inclusive token ranges of the chunks of a prompt ([KVM] I_k)."""
    if prompt_tokens < 1 or chunk_tokens < 1:
        raise ValueError("prompt and chunk lengths must be positive")
    n_chunks = -(-prompt_tokens // chunk_tokens)
    return [((k - 1) * chunk_tokens, min(k * chunk_tokens, prompt_tokens) - 1) for k in range(1, n_chunks + 1)]


def visible(history, chunk):
    """Boolean mask [chunk, history + chunk]: row j (position history + j) sees key t iff t <= history + j."""
    rows = np.arange(chunk)[:, None]
    keys = np.arange(history + chunk)[None, :]
    return keys <= history + rows


def visible_pairs(history, chunk):
    """Number of (query, key) pairs the mask lets through."""
    return int(visible(history, chunk).sum())


def chunk_attention(q, k, v, scale=None):
    """q [c, Hq, d]; k, v [n, Hkv, d] with n >= c (the last c rows are the chunk's own).

    Returns [c, Hq, d] float64: softmax(q K^T * scale + M) V per query head, with
    query head h reading KV head h // (Hq / Hkv) as in decode attention.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    c, num_q_heads, head_dim = q.shape
    n, num_kv_heads, _ = k.shape
    if c < 1 or n < c:
        raise ValueError("need 1 <= chunk length <= context length")
    if num_q_heads % num_kv_heads:
        raise ValueError("Hq must be a multiple of Hkv")
    group = num_q_heads // num_kv_heads
    if scale is None:
        scale = 1.0 / np.sqrt(head_dim)
    mask = visible(n - c, c)
    out = np.empty((c, num_q_heads, head_dim), dtype=np.float64)
    for h in range(num_q_heads):
        g = h // group
        s = (q[:, h, :] @ k[:, g, :].T) * scale  # [c, n]
        s = np.where(mask, s, -np.inf)
        w = np.exp(s - s.max(axis=1, keepdims=True))
        w /= w.sum(axis=1, keepdims=True)
        out[:, h, :] = w @ v[:, g, :]
    return out
