"""Closed-form sizes of a paged KV cache (test infrastructure; see oracle/__init__).

Integer arithmetic only, written from the definitions.
"""

from __future__ import annotations

from fractions import Fraction


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """Per-token KV footprint: one key and one value vector per KV head per layer.

    [KVM] Eq. 1; [BT] §01; [INF] §8.1.2.
    """
    return 2 * num_layers * num_kv_heads * head_dim * elem_bytes


def block_bytes(num_layers: int, num_kv_heads: int, block_size: int, head_dim: int,
                elem_bytes: int) -> int:
    """Bytes of one physical block holding ``block_size`` tokens of every layer and head.

    [KVM] PagedAttention virtual-memory model (M_block).
    """
    return block_size * kv_bytes_per_token(num_layers, num_kv_heads, head_dim, elem_bytes)


def blocks_needed(num_tokens: int, block_size: int) -> int:
    """ceil(S / B) blocks hold S tokens ([KVM] N_blocks; [INF] §8.3.1)."""
    return -(-num_tokens // block_size)


def tail_waste(num_tokens: int, block_size: int) -> int:
    """Unused slots in the last block: B * ceil(S/B) - S ([INF] §8.3.1; [KVM] Delta_tail)."""
    return block_size * blocks_needed(num_tokens, block_size) - num_tokens


def mean_tail_waste(block_size: int) -> Fraction:
    """Expected tail waste when S mod B is uniform over {0..B-1}, by enumeration.

    [KVM] block-size trade-off (the formula is rendered by the Russian
    translation; the Chinese extraction of the same line is garbled).
    """
    total = sum(tail_waste(r, block_size) for r in range(block_size))
    return Fraction(total, block_size)


def translate(position: int, block_size: int, table) -> tuple:
    """Logical position t -> (physical block, slot) = (table[t // B], t mod B). [BT] §03."""
    j, r = divmod(position, block_size)
    return table[j], r


def reload_seconds(num_tokens: int, bytes_per_token: int, link_bytes_per_s: float) -> float:
    """Time to stream a sequence's KV state over the host link: S * m_token / B_link.

    [KVM] evict-versus-swap analysis, T_reload; a round trip (out and back) takes twice this.
    """
    return num_tokens * bytes_per_token / link_bytes_per_s


def recompute_seconds(n_params: float, num_tokens: int, flops_per_s: float) -> float:
    """Time to rebuild the state by a prefill pass, linear term only: 2 P S / R_prefill.

    [KVM] evict-versus-swap analysis, T_recomp (the 4 L S^2 d_model attention term is
    dropped there for contexts up to about 32K tokens; so here).
    """
    return 2 * n_params * num_tokens / flops_per_s
