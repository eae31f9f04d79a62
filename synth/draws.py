"""Seeded random draws for the synthetic workloads.

Every tensor is drawn as float32 N(0,1) from numpy's PCG64 generator seeded by
a tuple ``(seed, tag, *index)`` and then stored either as float32 or rounded
to bfloat16 (round to nearest, ties to even).  Values are returned as raw bit
patterns (uint32 / uint16) so that byte-exact comparisons are possible, and
``bits_to_f64`` widens them exactly (every bf16 and fp32 value is an fp64
value).

Token K/V rows are drawn in chunks of ``CHUNK`` tokens so that a consumer that
needs only a few tokens of a long sequence (the oracle's sampled checks) can
regenerate exactly those chunks without drawing the whole sequence.
"""

from __future__ import annotations

import numpy as np

F32 = "f32"
BF16 = "bf16"

# Tags keep the streams of different tensors independent.
TAG_Q = 1
TAG_K = 2
TAG_V = 3
TAG_BACKGROUND = 4
TAG_QCHUNK = 5  # queries of multi-query (chunk / verification) attention

# Tokens per generator chunk for K/V rows.
CHUNK = 1024


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); finite inputs only."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # finite inputs: u + 0x8000 stays below 2**32, so uint32 arithmetic is exact
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bits_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored bit patterns to float64."""
    if dtype == F32:
        return np.asarray(bits, dtype=np.uint32).view(np.float32).astype(np.float64)
    if dtype == BF16:
        u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
        return u32.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def storage_np_dtype(dtype: str):
    return {F32: np.uint32, BF16: np.uint16}[dtype]


def normal_bits(seed: int, tag: int, index: tuple, shape, dtype: str) -> np.ndarray:
    """N(0,1) float32 draws of ``shape`` stored in ``dtype``, as raw bits."""
    rng = np.random.default_rng([int(seed), int(tag), *[int(i) for i in index]])
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == F32:
        return x.view(np.uint32)
    return f32_to_bf16_bits(x)


def token_rows(seed: int, tag: int, layer: int, writer: int, positions: np.ndarray,
               num_kv_heads: int, head_dim: int, dtype: str) -> np.ndarray:
    """K or V rows ``[len(positions), Hkv, d]`` for tokens written by ``writer``.

    The value of the token at ``position`` written by sequence ``writer`` in
    ``layer`` is row ``position % CHUNK`` of chunk ``position // CHUNK`` of that
    (layer, writer) stream, so any subset of positions can be regenerated
    independently.
    """
    positions = np.asarray(positions, dtype=np.int64)
    out = np.empty((positions.size, num_kv_heads, head_dim), dtype=storage_np_dtype(dtype))
    if positions.size == 0:
        return out
    chunks = positions // CHUNK
    for c in np.unique(chunks):
        sel = np.nonzero(chunks == c)[0]
        block = normal_bits(seed, tag, (layer, writer, int(c)), (CHUNK, num_kv_heads, head_dim), dtype)
        out[sel] = block[positions[sel] % CHUNK]
    return out


def free_order(seed: int, num_blocks: int) -> np.ndarray:
    """Initial free-list order: a seeded permutation of the block ids."""
    return np.random.default_rng(int(seed) + 1000).permutation(num_blocks).astype(np.int32)


def host_free_order(seed: int, num_frames: int) -> np.ndarray:
    """Initial order of the host frame free list: a seeded permutation of the frame ids."""
    return np.random.default_rng(int(seed) + 2000).permutation(num_frames).astype(np.int32)
