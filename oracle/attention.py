"""Single-query decode attention in float64 (test infrastructure; see oracle/__init__).

For one decode query q (Hq heads of dim d) over a context of n tokens whose
keys and values were gathered through the block table ([BT] §06-§07):

    s_t   = q_h . k_t / sqrt(d)                 for t = 0 .. n-1
    w     = exp(s - max s) / sum exp(s - max s)
    out_h = sum_t w_t v_t

with query head h reading KV head g = h // (Hq / Hkv): grouped-query attention
lets several query heads share one KV head ([BT] §06; [KVM] Eq. 1 context).
The grouping is contiguous, the plainest reading of the pages.  There is no
mask: the single decode query sees every cached position 0..n-1, its own
token included ([BT] §07 attends positions 0..i).

The split-K form computes, for each partition of the context, the running
maximum m, the sum l of exp(s - m) and the unnormalised o = sum exp(s - m) v,
then folds partitions together with the recurrences of [KVM] (chunked prefill
mechanism): m_new = max(m_prev, m_blk), l_new = l_prev e^(m_prev - m_new) +
l_blk e^(m_blk - m_new), O_new likewise; the output is O / l.
"""

from __future__ import annotations

import numpy as np


def decode_attention(q, k, v, scale=None):
    """q [Hq, d], k and v [n, Hkv, d] (float64) -> out [Hq, d] float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    num_q_heads, head_dim = q.shape
    n, num_kv_heads, _ = k.shape
    if n < 1:
        raise ValueError("a decode query needs at least one cached token")
    if num_q_heads % num_kv_heads:
        raise ValueError("Hq must be a multiple of Hkv")
    group = num_q_heads // num_kv_heads
    if scale is None:
        scale = 1.0 / np.sqrt(head_dim)
    out = np.empty((num_q_heads, head_dim), dtype=np.float64)
    for h in range(num_q_heads):
        g = h // group
        s = (k[:, g, :] @ q[h]) * scale
        w = np.exp(s - s.max())
        w /= w.sum()
        out[h] = w @ v[:, g, :]
    return out


def partition_stats(q, k, v, scale=None):
    """(m [Hq], l [Hq], o [Hq, d]) of one context partition, o unnormalised."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    num_q_heads, head_dim = q.shape
    num_kv_heads = k.shape[1]
    group = num_q_heads // num_kv_heads
    if scale is None:
        scale = 1.0 / np.sqrt(head_dim)
    m = np.empty(num_q_heads)
    l = np.empty(num_q_heads)
    o = np.empty((num_q_heads, head_dim))
    for h in range(num_q_heads):
        g = h // group
        s = (k[:, g, :] @ q[h]) * scale
        m[h] = s.max()
        e = np.exp(s - m[h])
        l[h] = e.sum()
        o[h] = e @ v[:, g, :]
    return m, l, o


def merge_partitions(parts):
    """Fold [(m, l, o), ...] with the running-max recurrences; return (m, l, o)."""
    m_run, l_run, o_run = parts[0]
    for m_blk, l_blk, o_blk in parts[1:]:
        m_new = np.maximum(m_run, m_blk)
        a = np.exp(m_run - m_new)
        b = np.exp(m_blk - m_new)
        l_run = l_run * a + l_blk * b
        o_run = o_run * a[:, None] + o_blk * b[:, None]
        m_run = m_new
    return m_run, l_run, o_run


def split_k_attention(q, k, v, partition_tokens, scale=None):
    """Decode attention computed per partition of ``partition_tokens`` and merged."""
    n = k.shape[0]
    parts = [partition_stats(q, k[a:a + partition_tokens], v[a:a + partition_tokens], scale)
             for a in range(0, n, partition_tokens)]
    _, l, o = merge_partitions(parts)
    return o / l[:, None]

