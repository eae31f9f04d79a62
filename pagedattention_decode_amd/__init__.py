"""Paged KV cache with decode and multi-query (chunked prefill / draft
verification) attention for MI355X (gfx950).

The work is done by ``libpagedkv.so`` (C ABI in ``include/pagedkv.h``): a C++
host block manager and hand-written HIP kernels.  :mod:`.binding` exposes the
C functions under the same names; :mod:`.pool` adds a small owner object that
allocates the pool buffers with torch and keeps the handle.
"""

from . import binding  # noqa: F401
from .binding import (  # noqa: F401
    KV_BF16,
    KV_F32,
    KV_Q4_0,
    KV_Q8_0,
    KV_KERNEL_AUTO,
    KV_KERNEL_GENERIC,
    KV_KERNEL_MFMA,
    KVError,
    KVOutOfBlocks,
    attention_options,
    copy_blocks,
    kv_append_slots,
    kv_get_block_tables,
    kv_pool_check,
    kv_pool_create,
    kv_pool_destroy,
    kv_pool_required_bytes,
    kv_seq_add,
    kv_seq_fork,
    kv_seq_release,
    paged_attention_decode,
    paged_attention_prefill,
    paged_attention_workspace_bytes,
    paged_prefill_workspace_bytes,
    reshape_and_cache,
)
from .pool import PagedKVPool  # noqa: F401
