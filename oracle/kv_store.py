"""Logical K/V pool of the oracle (test infrastructure; see oracle/__init__).

Values are kept as raw stored bit patterns in the order the block-table page
gives as its example layout, ``[layer][block][slot][kv_head][dim]`` ([BT] §06),
so that byte-exact comparisons need no rounding.  Blocks are materialised
lazily: a block that was never written holds the ``background`` pattern (zeros
by default), so large pools cost only what is written.

* ``write``   puts token rows at flat slots ``slot = block * B + offset``
              ([BT] §03-§04; [KVM] paged KV allocation: the new token's key and
              value go to T[l] at offset o); negative slots are skipped.
* ``copy_blocks`` replaces ``dst`` by a copy of ``src`` in every layer
              ([KVM] CoW branching: the shared block's B tokens are copied).
* ``gather``  returns the first ``n`` token rows of a sequence by walking its
              block table ([BT] §06: block_table[seq, t // B], then t % B).
* ``to_host`` / ``from_host`` copy whole blocks (every layer) to host frames and
              back ([KVM] asynchronous paged swap: a block's bytes move
              unchanged between the tiers).
"""

from __future__ import annotations

import numpy as np


class KVStore:
    def __init__(self, num_layers, num_blocks, block_size, num_kv_heads, head_dim,
                 storage_dtype, background=None, layers=None):
        self.num_layers = num_layers
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.num_kv_heads = num_kv_heads
        self.head_dim = head_dim
        self.storage_dtype = storage_dtype
        # background(layer, which, block) -> [B, Hkv, d] bits; which is "k" or "v"
        self.background = background
        # only these layers are materialised (None = all)
        self.layers = None if layers is None else set(layers)
        self.k: dict = {}
        self.v: dict = {}

    def _tracked(self, layer) -> bool:
        return self.layers is None or layer in self.layers

    def _block(self, store, which, layer, block, create):
        key = (layer, block)
        blk = store.get(key)
        if blk is None:
            if self.background is not None:
                blk = np.array(self.background(layer, which, block), dtype=self.storage_dtype)
            else:
                blk = np.zeros((self.block_size, self.num_kv_heads, self.head_dim),
                               dtype=self.storage_dtype)
            if create:
                store[key] = blk
        return blk

    def write(self, layer, slots, k_rows, v_rows) -> None:
        if not self._tracked(layer):
            return
        for i, slot in enumerate(slots):
            if slot < 0:
                continue
            block, offset = divmod(int(slot), self.block_size)
            self._block(self.k, "k", layer, block, True)[offset] = k_rows[i]
            self._block(self.v, "v", layer, block, True)[offset] = v_rows[i]

    def copy_blocks(self, pairs) -> None:
        for layer in range(self.num_layers):
            if not self._tracked(layer):
                continue
            for src, dst in pairs:
                self.k[(layer, dst)] = self._block(self.k, "k", layer, src, False).copy()
                self.v[(layer, dst)] = self._block(self.v, "v", layer, src, False).copy()

    def block(self, which, layer, block) -> np.ndarray:
        store = self.k if which == "k" else self.v
        return self._block(store, which, layer, block, False)

    def to_host(self, pairs) -> None:
        """(block, frame) pairs: frame := block, in every tracked layer."""
        if not hasattr(self, "host_k"):
            self.host_k, self.host_v = {}, {}
        for layer in range(self.num_layers):
            if not self._tracked(layer):
                continue
            for block, frame in pairs:
                self.host_k[(layer, frame)] = self._block(self.k, "k", layer, block, False).copy()
                self.host_v[(layer, frame)] = self._block(self.v, "v", layer, block, False).copy()

    def from_host(self, pairs) -> None:
        """(frame, block) pairs: block := frame, in every tracked layer."""
        for layer in range(self.num_layers):
            if not self._tracked(layer):
                continue
            for frame, block in pairs:
                self.k[(layer, block)] = self.host_k[(layer, frame)].copy()
                self.v[(layer, block)] = self.host_v[(layer, frame)].copy()

    def host_block(self, which, layer, frame) -> np.ndarray:
        return (self.host_k if which == "k" else self.host_v)[(layer, frame)]

    def gather(self, layer, table, n):
        """K and V rows [n, Hkv, d] of a sequence of length n with block table ``table``."""
        k = np.empty((n, self.num_kv_heads, self.head_dim), dtype=self.storage_dtype)
        v = np.empty_like(k)
        for t in range(0, n, self.block_size):
            j = t // self.block_size
            take = min(self.block_size, n - t)
            k[t:t + take] = self.block("k", layer, table[j])[:take]
            v[t:t + take] = self.block("v", layer, table[j])[:take]
        return k, v
