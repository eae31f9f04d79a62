"""Owner object for one pool: torch allocates the K/V buffers, the library keeps
the host block manager.  Marshalling only; see include/pagedkv.h for semantics.
"""

from __future__ import annotations

import numpy as np

from . import binding as B


class PagedKVPool:
    def __init__(self, num_layers, num_blocks, block_size, num_kv_heads, head_dim, dtype="bf16",
                 free_order=None, device="cuda", allocate=True):
        self.dtype = dtype
        code = B.DTYPE_CODES[dtype]
        self.cfg = B.make_config(num_layers, num_blocks, block_size, num_kv_heads, head_dim, code)
        self.num_layers, self.num_blocks, self.block_size = num_layers, num_blocks, block_size
        self.num_kv_heads, self.head_dim = num_kv_heads, head_dim
        kb, vb = B.kv_pool_required_bytes(self.cfg)
        self.k_cache = self.v_cache = None
        if allocate:
            import torch
            # raw storage; elements are viewed per dtype by the caller when needed
            self.k_cache = torch.empty(kb, dtype=torch.uint8, device=device)
            self.v_cache = torch.empty(vb, dtype=torch.uint8, device=device)
        self.handle = B.kv_pool_create(self.cfg, self.k_cache if allocate else 0,
                                       self.v_cache if allocate else 0, free_order)

    def close(self):
        if self.handle is not None:
            B.kv_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- host block manager ----------------------------------------------
    def add(self, seq):
        B.kv_seq_add(self.handle, seq)

    def fork(self, parent, child):
        B.kv_seq_fork(self.handle, parent, child)

    def append(self, seq_ids, counts=None):
        return B.kv_append_slots(self.handle, seq_ids, counts)

    def tables(self, seq_ids, max_blocks):
        return B.kv_get_block_tables(self.handle, seq_ids, max_blocks)

    def info(self, seq):
        return B.kv_seq_info(self.handle, seq)

    def release(self, seq, stream=None):
        B.kv_seq_release(self.handle, seq, stream)

    def release_fenced(self, seq, fence):
        B.kv_seq_release_fenced(self.handle, seq, fence)

    def retire(self, completed):
        B.kv_pool_retire(self.handle, completed)

    def reclaim(self, wait=False):
        B.kv_pool_reclaim(self.handle, wait)

    def stats(self):
        return B.kv_pool_stats(self.handle)

    def free_list(self):
        return B.kv_pool_free_list(self.handle, self.num_blocks)

    def refcounts(self):
        return B.kv_pool_refcounts(self.handle, self.num_blocks)

    def check(self):
        B.kv_pool_check(self.handle)

    # -- device operations ---------------------------------------------------
    def cache(self, layer, k_new, v_new, slot_mapping, stream=None):
        B.reshape_and_cache(self.handle, layer, k_new, v_new, slot_mapping, stream)

    def copy(self, pairs, stream=None):
        B.copy_blocks(self.handle, pairs, stream)

    def workspace_bytes(self, n_seqs, num_q_heads, max_blocks, opts=None):
        return B.paged_attention_workspace_bytes(self.handle, n_seqs, num_q_heads, max_blocks, opts)

    def decode(self, layer, q, out, block_tables, context_lens, num_q_heads, opts=None, workspace=None,
               stream=None):
        B.paged_attention_decode(self.handle, layer, q, out, block_tables, context_lens, num_q_heads, opts,
                                 workspace, stream)

    def decode_static(self, layer, q, out, block_tables, context_lens, num_q_heads, opts=None, stream=None):
        B.paged_attention_decode_static(self.handle, layer, q, out, block_tables, context_lens, num_q_heads, opts,
                                        stream)

    def prefill_workspace_bytes(self, n_seqs, total_q, max_q_len, num_q_heads, max_blocks, opts=None):
        return B.paged_prefill_workspace_bytes(self.handle, n_seqs, total_q, max_q_len, num_q_heads, max_blocks, opts)

    def prefill(self, layer, q, out, q_indptr, block_tables, context_lens, max_q_len, num_q_heads, opts=None,
                workspace=None, stream=None):
        B.paged_attention_prefill(self.handle, layer, q, out, q_indptr, block_tables, context_lens, max_q_len,
                                  num_q_heads, opts, workspace, stream)

    def shared_prefix_plan(self, seq_ids):
        return B.kv_shared_prefix_plan(self.handle, seq_ids)

    def cascade_workspace_bytes(self, n_seqs, n_groups, max_group, num_q_heads, max_blocks, opts=None):
        return B.paged_attention_cascade_workspace_bytes(self.handle, n_seqs, n_groups, max_group, num_q_heads,
                                                         max_blocks, opts)

    def decode_cascade(self, layer, q, out, block_tables, context_lens, num_q_heads, group_start, shared_blocks,
                       max_group, opts=None, workspace=None, stream=None):
        B.paged_attention_decode_cascade(self.handle, layer, q, out, block_tables, context_lens, num_q_heads,
                                         group_start, shared_blocks, max_group, opts, workspace, stream)

    # -- host tier ----------------------------------------------------------
    def attach_host(self, n_frames, free_order=None, staging_bytes=64 << 20):
        """Pinned host frames (allocated here when the pool owns device memory) and a
        device staging buffer of whole frames (at least one)."""
        self.frame_bytes = B.kv_host_frame_bytes(self.handle)
        self.n_frames = n_frames
        self.host_frames = self.staging = None
        if self.k_cache is not None:
            import torch
            self.host_frames = torch.empty(n_frames * self.frame_bytes, dtype=torch.uint8, pin_memory=True)
            frames = max(1, staging_bytes // self.frame_bytes)
            self.staging = torch.empty(frames * self.frame_bytes, dtype=torch.uint8, device=self.k_cache.device)
        B.kv_pool_attach_host(self.handle, self.host_frames, n_frames, free_order)

    def swap_out(self, seq, stream=None):
        return B.kv_seq_swap_out(self.handle, seq, self.staging, stream)

    def swap_in(self, seq, stream=None):
        return B.kv_seq_swap_in(self.handle, seq, self.staging, stream)

    def swap_out_fenced(self, seq, fence):
        return B.kv_seq_swap_out_fenced(self.handle, seq, fence)

    def swap_in_fenced(self, seq, fence):
        return B.kv_seq_swap_in_fenced(self.handle, seq, fence)

    def swap_copy(self, pairs, direction, stream=None):
        B.kv_swap_copy(self.handle, pairs, direction, self.staging, stream)

    def residency(self, seq):
        return B.kv_seq_residency(self.handle, seq)

    def host_free_list(self):
        return B.kv_host_free_list(self.handle, self.n_frames)

    # -- prefix cache --------------------------------------------------------
    def prefix_match(self, tokens):
        return B.kv_prefix_match(self.handle, tokens)

    def attach_prefix(self, seq, tokens):
        return B.kv_seq_attach_prefix(self.handle, seq, tokens)

    def prefix_insert(self, seq, tokens):
        return B.kv_prefix_insert(self.handle, seq, tokens)

    def prefix_evict(self, target_free, stream=None, fence=None):
        return B.kv_prefix_evict(self.handle, target_free, stream, fence)

    def prefix_stats(self):
        return B.kv_prefix_stats(self.handle)

    # -- raw views for tests -------------------------------------------------
    def raw(self, which):
        """The K or V buffer as a flat tensor of stored bit patterns (bytes for a quantised pool)."""
        import torch
        buf = self.k_cache if which == "k" else self.v_cache
        if self.dtype in ("q8_0", "q4_0"):
            return buf
        return buf.view(torch.int16 if self.dtype == "bf16" else torch.int32)


def np_storage(dtype):
    return np.uint16 if dtype == "bf16" else np.uint32
