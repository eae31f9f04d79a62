"""ctypes binding of libpagedkv.so (include/pagedkv.h).

Argument marshalling only: every function has the C name, converts torch
tensors to device pointers (and the current HIP stream when none is given),
numpy arrays to host pointers, and turns a non-OK status into an exception
carrying kv_last_error().  All computation happens in the library.  Loading
fails loudly when the library has not been built.
"""

from __future__ import annotations

import ctypes as C
import os

import numpy as np

from .build import LIB_PATH

KV_OK, KV_ERR_OOM, KV_ERR_INVALID, KV_ERR_STATE, KV_ERR_HIP, KV_ERR_UNSUPPORTED = range(6)
KV_F32, KV_BF16, KV_Q8_0, KV_Q4_0 = 0, 1, 2, 3
DTYPE_CODES = {"f32": KV_F32, "bf16": KV_BF16, "q8_0": KV_Q8_0, "q4_0": KV_Q4_0}
KV_KERNEL_AUTO, KV_KERNEL_GENERIC, KV_KERNEL_MFMA, KV_KERNEL_MFMA_STAGED_TABLE, KV_KERNEL_VALU = 0, 1, 2, 3, 4


class KVError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"[status {status}] {message}")
        self.status = status


class KVOutOfBlocks(KVError, MemoryError):
    pass


class KVArgumentError(KVError, ValueError):
    """A tensor argument whose device, element type, shape or layout does not
    match the call (found by the binding before the library is called)."""

    def __init__(self, message):
        super().__init__(KV_ERR_INVALID, message)


class kv_pool_config(C.Structure):
    _fields_ = [("num_layers", C.c_int32), ("num_blocks", C.c_int32), ("block_size", C.c_int32),
                ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("dtype", C.c_int32)]


class kv_pool_stats_t(C.Structure):
    _fields_ = [("n_free", C.c_int32), ("n_allocated", C.c_int32), ("n_shared", C.c_int32),
                ("n_pending", C.c_int32), ("n_seqs", C.c_int32), ("n_tokens", C.c_int64),
                ("n_table_refs", C.c_int64)]


class kv_timing_events(C.Structure):
    _fields_ = [("start", C.c_void_p), ("kernel_stop", C.c_void_p), ("stop", C.c_void_p)]


class kv_attention_options(C.Structure):
    _fields_ = [("scale", C.c_float), ("partition_tokens", C.c_int32), ("kernel", C.c_int32),
                ("timing", C.POINTER(kv_timing_events))]


_P = C.c_void_p
_I32 = C.c_int32
_I64 = C.c_int64
_U64 = C.c_uint64

# name -> (restype, argtypes); the exported surface of include/pagedkv.h
SIGNATURES = {
    "kv_pool_required_bytes": (_I32, [C.POINTER(kv_pool_config), C.POINTER(_U64), C.POINTER(_U64)]),
    "kv_pool_create": (_I32, [C.POINTER(kv_pool_config), _P, _P, _P, C.POINTER(_P)]),
    "kv_pool_destroy": (None, [_P]),
    "kv_seq_add": (_I32, [_P, _I64]),
    "kv_seq_fork": (_I32, [_P, _I64, _I64]),
    "kv_append_slots": (_I32, [_P, _I32, _P, _P, _P, _I64, _P, _I32, C.POINTER(_I32)]),
    "kv_get_block_tables": (_I32, [_P, _I32, _P, _I32, _P, _P]),
    "kv_seq_info": (_I32, [_P, _I64, C.POINTER(_I32), C.POINTER(_I32)]),
    "kv_seq_release": (_I32, [_P, _I64, _P]),
    "kv_seq_release_fenced": (_I32, [_P, _I64, _U64]),
    "kv_pool_retire": (_I32, [_P, _U64]),
    "kv_pool_reclaim": (_I32, [_P, _I32]),
    "kv_pool_stats": (_I32, [_P, C.POINTER(kv_pool_stats_t)]),
    "kv_pool_get_config": (_I32, [_P, C.POINTER(kv_pool_config)]),
    "kv_pool_free_list": (_I32, [_P, _I32, _P, C.POINTER(_I32)]),
    "kv_pool_refcounts": (_I32, [_P, _P]),
    "kv_pool_check": (_I32, [_P]),
    "kv_last_error": (C.c_char_p, []),
    "reshape_and_cache": (_I32, [_P, _I32, _P, _P, _P, _I32, _P]),
    "copy_blocks": (_I32, [_P, _P, _I32, _P]),
    "paged_attention_workspace_bytes": (_U64, [_P, _I32, _I32, _I32, C.POINTER(kv_attention_options)]),
    "paged_attention_decode": (_I32, [_P, _I32, _P, _P, _P, _P, _I32, _I32, _I32,
                                      C.POINTER(kv_attention_options), _P, _U64, _P]),
    "paged_attention_static_scratch_bytes": (_U64, []),
    "paged_attention_decode_static": (_I32, [_P, _I32, _P, _P, _P, _P, _I32, _I32, _I32,
                                             C.POINTER(kv_attention_options), _P]),
    "kv_prefix_match": (_I32, [_P, _P, _I32, C.POINTER(_I32), C.POINTER(_I32)]),
    "kv_seq_attach_prefix": (_I32, [_P, _I64, _P, _I32, C.POINTER(_I32)]),
    "kv_prefix_insert": (_I32, [_P, _I64, _P, _I32, C.POINTER(_I32)]),
    "kv_prefix_evict": (_I32, [_P, _I32, _P, _P, _I32, C.POINTER(_I32)]),
    "kv_prefix_evict_fenced": (_I32, [_P, _I32, _U64, _P, _I32, C.POINTER(_I32)]),
    "kv_prefix_stats": (_I32, [_P, C.POINTER(_I32), C.POINTER(_I32), C.POINTER(_I32)]),
    "kv_shared_prefix_plan": (_I32, [_P, _I32, _P, _P, _P, C.POINTER(_I32)]),
    "paged_attention_cascade_workspace_bytes": (_U64, [_P, _I32, _I32, _I32, _I32, _I32,
                                                       C.POINTER(kv_attention_options)]),
    "paged_attention_decode_cascade": (_I32, [_P, _I32, _P, _P, _P, _P, _I32, _I32, _I32, _P, _P, _I32, _I32,
                                              C.POINTER(kv_attention_options), _P, _U64, _P]),
    "kv_host_frame_bytes": (_U64, [_P]),
    "kv_pool_attach_host": (_I32, [_P, _P, _I32, _P]),
    "kv_seq_swap_out": (_I32, [_P, _I64, _P, _U64, _P, _P, _I32, C.POINTER(_I32)]),
    "kv_seq_swap_in": (_I32, [_P, _I64, _P, _U64, _P, _P, _I32, C.POINTER(_I32)]),
    "kv_seq_swap_out_fenced": (_I32, [_P, _I64, _U64, _P, _I32, C.POINTER(_I32)]),
    "kv_seq_swap_in_fenced": (_I32, [_P, _I64, _U64, _P, _I32, C.POINTER(_I32)]),
    "kv_swap_copy": (_I32, [_P, _P, _I32, _I32, _P, _U64, _P]),
    "kv_seq_residency": (_I32, [_P, _I64, _I32, _P, _P, C.POINTER(_I32)]),
    "kv_host_free_list": (_I32, [_P, _I32, _P, C.POINTER(_I32)]),
    "paged_prefill_workspace_bytes": (_U64, [_P, _I32, _I32, _I32, _I32, _I32, C.POINTER(kv_attention_options)]),
    "paged_attention_prefill": (_I32, [_P, _I32, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                       C.POINTER(kv_attention_options), _P, _U64, _P]),
}

_lib = None


def lib_path():
    """The library to load: libpagedkv.so, or the file named by PAGEDKV_LIBRARY
    (the host-only sanitizer build of the CPU tests, whose device entry points
    all fail with KV_ERR_UNSUPPORTED)."""
    return os.environ.get("PAGEDKV_LIBRARY") or LIB_PATH


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python -m pagedattention_decode_amd.build`")
        handle = C.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status):
    if status != KV_OK:
        msg = lib().kv_last_error().decode(errors="replace")
        if status == KV_ERR_OOM:
            raise KVOutOfBlocks(status, msg)
        raise KVError(status, msg)


def _host(arr, dtype):
    a = np.ascontiguousarray(arr, dtype=dtype)
    return a, a.ctypes.data_as(C.c_void_p)


def _dev(t):
    """Device pointer of a contiguous torch tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise KVArgumentError("device tensors must be contiguous")
    return C.c_void_p(t.data_ptr())


# -- argument checks ----------------------------------------------------------
# The C ABI takes raw pointers, so a tensor of the wrong element type or shape
# would be read out of bounds or misread; these checks refuse such arguments
# before the call.  Tensors holding bf16 / f32 values may be given in any
# torch type of the same element size (the tests pass raw bit patterns as
# int16 / int32).

_configs = {}


def kv_pool_get_config(pool):
    key = pool.value if isinstance(pool, C.c_void_p) else int(pool)
    cfg = _configs.get(key)
    if cfg is None:
        cfg = kv_pool_config()
        _check(lib().kv_pool_get_config(pool, C.byref(cfg)))
        _configs[key] = cfg
    return cfg


def _forget_config(pool):
    _configs.pop(pool.value if isinstance(pool, C.c_void_p) else int(pool), None)


def _row_bytes(cfg):
    """Element size of new K/V rows, queries and outputs for this pool: 4 for an
    f32 pool, 2 (bf16) otherwise."""
    return 4 if cfg.dtype == KV_F32 else 2


def _need(cond, msg):
    if not cond:
        raise KVArgumentError(msg)


def _device_tensor(t, name, ndim=None, elem=None, dtype=None, shape=None):
    import torch
    _need(isinstance(t, torch.Tensor), f"{name} must be a torch tensor")
    _need(t.is_cuda, f"{name} must be on the GPU (it is on {t.device})")
    _need(t.is_contiguous(), f"{name} must be contiguous")
    if dtype is not None:
        _need(t.dtype == dtype, f"{name} must be {dtype} (it is {t.dtype})")
    if elem is not None:
        _need(t.element_size() == elem and not t.is_complex(),
              f"{name} must have {elem}-byte elements (it has {t.dtype})")
    if ndim is not None:
        _need(t.dim() == ndim, f"{name} must have {ndim} dimensions (shape {tuple(t.shape)})")
    if shape is not None:
        _need(tuple(t.shape) == tuple(shape), f"{name} must have shape {tuple(shape)} (it has {tuple(t.shape)})")


def _rows(pool, t, name, n, heads):
    """A [n, heads, d] tensor of the pool's row element type."""
    cfg = kv_pool_get_config(pool)
    _device_tensor(t, name, ndim=3, elem=_row_bytes(cfg), shape=(n, heads, cfg.head_dim))


def _tables(block_tables, context_lens, n=None):
    import torch
    _device_tensor(block_tables, "block_tables", ndim=2, dtype=torch.int32)
    n = block_tables.shape[0] if n is None else n
    _need(block_tables.shape[0] == n, f"block_tables must have {n} rows")
    _device_tensor(context_lens, "context_lens", dtype=torch.int32, shape=(n,))


def _workspace(ws):
    if ws is not None:
        _device_tensor(ws, "workspace")


def _stream(stream):
    if stream is None:
        import torch
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return C.c_void_p(stream)
    return C.c_void_p(stream.cuda_stream)


# -- pool -------------------------------------------------------------------

def make_config(num_layers, num_blocks, block_size, num_kv_heads, head_dim, dtype):
    return kv_pool_config(num_layers, num_blocks, block_size, num_kv_heads, head_dim, dtype)


def kv_pool_required_bytes(cfg):
    kb, vb = _U64(), _U64()
    _check(lib().kv_pool_required_bytes(C.byref(cfg), C.byref(kb), C.byref(vb)))
    return kb.value, vb.value


def kv_pool_create(cfg, k_cache, v_cache, initial_free_order=None):
    """k_cache / v_cache: torch tensors (device) or raw integer addresses."""
    order = None
    ptr = None
    if initial_free_order is not None:
        order, ptr = _host(initial_free_order, np.int32)
    out = _P()
    kp = k_cache if isinstance(k_cache, int) or k_cache is None else k_cache.data_ptr()
    vp = v_cache if isinstance(v_cache, int) or v_cache is None else v_cache.data_ptr()
    _check(lib().kv_pool_create(C.byref(cfg), kp, vp, ptr, C.byref(out)))
    del order
    return out


def kv_pool_destroy(pool):
    _forget_config(pool)
    lib().kv_pool_destroy(pool)


def kv_seq_add(pool, seq_id):
    _check(lib().kv_seq_add(pool, int(seq_id)))


def kv_seq_fork(pool, parent, child):
    _check(lib().kv_seq_fork(pool, int(parent), int(child)))


def kv_append_slots(pool, seq_ids, n_new=None):
    """Returns (slot_mapping int64[sum n_new], cow_pairs int64[k, 2])."""
    seq_ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
    n = seq_ids.size
    n_new = np.ones(n, np.int32) if n_new is None else np.ascontiguousarray(n_new, dtype=np.int32)
    total = int(n_new.sum(dtype=np.int64))
    slots = np.empty(max(total, 1), np.int64)
    pairs = np.empty((max(n, 1), 2), np.int64)
    n_cow = _I32()
    _check(lib().kv_append_slots(pool, n, seq_ids.ctypes.data_as(_P), n_new.ctypes.data_as(_P),
                                 slots.ctypes.data_as(_P), total, pairs.ctypes.data_as(_P),
                                 max(n, 1), C.byref(n_cow)))
    return slots[:total], pairs[:n_cow.value].copy()


def kv_get_block_tables(pool, seq_ids, max_blocks):
    seq_ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
    n = seq_ids.size
    tables = np.empty((n, max_blocks), np.int32)
    lens = np.empty(n, np.int32)
    _check(lib().kv_get_block_tables(pool, n, seq_ids.ctypes.data_as(_P), max_blocks,
                                     tables.ctypes.data_as(_P), lens.ctypes.data_as(_P)))
    return tables, lens


def kv_seq_info(pool, seq_id):
    length, nb = _I32(), _I32()
    _check(lib().kv_seq_info(pool, int(seq_id), C.byref(length), C.byref(nb)))
    return length.value, nb.value


def kv_seq_release(pool, seq_id, stream=None):
    _check(lib().kv_seq_release(pool, int(seq_id), _stream(stream)))


def kv_seq_release_fenced(pool, seq_id, fence):
    _check(lib().kv_seq_release_fenced(pool, int(seq_id), int(fence)))


def kv_pool_retire(pool, completed_fence):
    _check(lib().kv_pool_retire(pool, int(completed_fence)))


def kv_pool_reclaim(pool, wait=False):
    _check(lib().kv_pool_reclaim(pool, 1 if wait else 0))


def kv_pool_stats(pool):
    s = kv_pool_stats_t()
    _check(lib().kv_pool_stats(pool, C.byref(s)))
    return {f: getattr(s, f) for f, _ in kv_pool_stats_t._fields_}


def kv_pool_free_list(pool, num_blocks):
    out = np.empty(max(num_blocks, 1), np.int32)
    n = _I32()
    _check(lib().kv_pool_free_list(pool, num_blocks, out.ctypes.data_as(_P), C.byref(n)))
    return out[:n.value].copy()


def kv_pool_refcounts(pool, num_blocks):
    out = np.empty(num_blocks, np.int32)
    _check(lib().kv_pool_refcounts(pool, out.ctypes.data_as(_P)))
    return out


def kv_pool_check(pool):
    _check(lib().kv_pool_check(pool))


def kv_last_error():
    return lib().kv_last_error().decode(errors="replace")


# -- device operations ----------------------------------------------------

def reshape_and_cache(pool, layer, k_new, v_new, slot_mapping, stream=None):
    """k_new, v_new: device [n, Hkv, d]; slot_mapping: device int64 [n]."""
    import torch
    _device_tensor(slot_mapping, "slot_mapping", ndim=1, dtype=torch.int64)
    n = int(slot_mapping.numel())
    cfg = kv_pool_get_config(pool)
    _rows(pool, k_new, "k_new", n, cfg.num_kv_heads)
    _rows(pool, v_new, "v_new", n, cfg.num_kv_heads)
    _check(lib().reshape_and_cache(pool, int(layer), _dev(k_new), _dev(v_new), _dev(slot_mapping), n,
                                   _stream(stream)))


def copy_blocks(pool, pairs, stream=None):
    """pairs: device int64 [k, 2] of (src, dst)."""
    if pairs is not None:
        import torch
        _device_tensor(pairs, "pairs", ndim=2, dtype=torch.int64)
        _need(pairs.shape[1] == 2, "pairs must have shape [k, 2]")
    n = int(pairs.shape[0]) if pairs is not None else 0
    _check(lib().copy_blocks(pool, _dev(pairs) if n else None, n, _stream(stream)))


def _event_handle(ev):
    if ev is None:
        return None
    if isinstance(ev, int):
        return ev
    h = int(ev.cuda_event)  # torch.cuda.Event: exists once it has been recorded
    if not h:
        raise ValueError("timing event has no HIP event yet: record it once before passing it")
    return h


def attention_options(scale=0.0, partition_tokens=0, kernel=KV_KERNEL_AUTO, timing=None):
    """timing: None or (start, kernel_stop, stop), each a torch.cuda.Event
    (already recorded once), a raw hipEvent_t or None (kv_timing_events)."""
    o = kv_attention_options(float(scale), int(partition_tokens), int(kernel))
    if timing is not None:
        start, kernel_stop, stop = timing
        o.timing = C.pointer(kv_timing_events(_event_handle(start), _event_handle(kernel_stop),
                                              _event_handle(stop)))
    return o


def paged_attention_workspace_bytes(pool, n_seqs, num_q_heads, max_blocks_per_seq, opts=None):
    return int(lib().paged_attention_workspace_bytes(pool, int(n_seqs), int(num_q_heads), int(max_blocks_per_seq),
                                                     C.byref(opts) if opts is not None else None))


def paged_attention_decode(pool, layer, q, out, block_tables, context_lens, num_q_heads, opts=None,
                           workspace=None, stream=None):
    """q, out: device [n, Hq, d]; block_tables: device int32 [n, max_blocks]; context_lens int32 [n]."""
    _tables(block_tables, context_lens)
    n_seqs, max_blocks = int(block_tables.shape[0]), int(block_tables.shape[1])
    _rows(pool, q, "q", n_seqs, num_q_heads)
    _rows(pool, out, "out", n_seqs, num_q_heads)
    _workspace(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().paged_attention_decode(pool, int(layer), _dev(q), _dev(out), _dev(block_tables),
                                        _dev(context_lens), n_seqs, max_blocks, int(num_q_heads),
                                        C.byref(opts) if opts is not None else None, _dev(workspace),
                                        ws_bytes, _stream(stream)))


def paged_attention_static_scratch_bytes():
    return int(lib().paged_attention_static_scratch_bytes())


def paged_attention_decode_static(pool, layer, q, out, block_tables, context_lens, num_q_heads, opts=None,
                                  stream=None):
    """paged_attention_decode with the library's static device scratch instead of a
    workspace: allocates nothing (arguments as for paged_attention_decode)."""
    _tables(block_tables, context_lens)
    n_seqs, max_blocks = int(block_tables.shape[0]), int(block_tables.shape[1])
    _rows(pool, q, "q", n_seqs, num_q_heads)
    _rows(pool, out, "out", n_seqs, num_q_heads)
    _check(lib().paged_attention_decode_static(pool, int(layer), _dev(q), _dev(out), _dev(block_tables),
                                               _dev(context_lens), n_seqs, max_blocks, int(num_q_heads),
                                               C.byref(opts) if opts is not None else None, _stream(stream)))


def paged_prefill_workspace_bytes(pool, n_seqs, total_q, max_q_len, num_q_heads, max_blocks_per_seq, opts=None):
    return int(lib().paged_prefill_workspace_bytes(pool, int(n_seqs), int(total_q), int(max_q_len), int(num_q_heads),
                                                   int(max_blocks_per_seq),
                                                   C.byref(opts) if opts is not None else None))


def paged_attention_prefill(pool, layer, q, out, q_indptr, block_tables, context_lens, max_q_len, num_q_heads,
                            opts=None, workspace=None, stream=None):
    """q, out: device [total_q, Hq, d]; q_indptr: device int32 [n + 1]; block_tables: device
    int32 [n, max_blocks]; context_lens: device int32 [n] (lengths after the chunk)."""
    import torch
    _tables(block_tables, context_lens)
    n_seqs, max_blocks = int(block_tables.shape[0]), int(block_tables.shape[1])
    _device_tensor(q, "q", ndim=3)
    total_q = int(q.shape[0])
    _rows(pool, q, "q", total_q, num_q_heads)
    _rows(pool, out, "out", total_q, num_q_heads)
    _device_tensor(q_indptr, "q_indptr", dtype=torch.int32, shape=(n_seqs + 1,))
    _workspace(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().paged_attention_prefill(pool, int(layer), _dev(q), _dev(out), _dev(q_indptr), _dev(block_tables),
                                         _dev(context_lens), n_seqs, total_q, int(max_q_len), max_blocks,
                                         int(num_q_heads), C.byref(opts) if opts is not None else None,
                                         _dev(workspace), ws_bytes, _stream(stream)))


# -- prefix cache ------------------------------------------------------------

def kv_prefix_match(pool, tokens):
    """(S_match, S_usable) of the longest cached prefix of ``tokens``."""
    t, tp = _host(tokens, np.int32)
    m, u = _I32(), _I32()
    _check(lib().kv_prefix_match(pool, tp, len(t), C.byref(m), C.byref(u)))
    return m.value, u.value


def kv_seq_attach_prefix(pool, seq_id, tokens):
    t, tp = _host(tokens, np.int32)
    c = _I32()
    _check(lib().kv_seq_attach_prefix(pool, int(seq_id), tp, len(t), C.byref(c)))
    return c.value


def kv_prefix_insert(pool, seq_id, tokens):
    t, tp = _host(tokens, np.int32)
    c = _I32()
    _check(lib().kv_prefix_insert(pool, int(seq_id), tp, len(t), C.byref(c)))
    return c.value


def kv_prefix_evict(pool, target_free, stream=None, fence=None, cap=1 << 16):
    """Evict; with ``fence`` given, the fenced form (0 = blocks free at once).
    Returns the evicted nodes' blocks in eviction order (at most ``cap``)."""
    n = _I32()
    out = np.empty(cap, np.int32)
    op = out.ctypes.data_as(C.c_void_p)
    if fence is not None:
        _check(lib().kv_prefix_evict_fenced(pool, int(target_free), int(fence), op, cap, C.byref(n)))
    else:
        _check(lib().kv_prefix_evict(pool, int(target_free), _stream(stream), op, cap, C.byref(n)))
    return out[:min(n.value, cap)].tolist()


def kv_prefix_stats(pool):
    a, b, c = _I32(), _I32(), _I32()
    _check(lib().kv_prefix_stats(pool, C.byref(a), C.byref(b), C.byref(c)))
    return {"n_nodes": a.value, "n_cached_blocks": b.value, "n_pinned": c.value}


# -- cascade decode over shared prefixes ---------------------------------------

def kv_shared_prefix_plan(pool, seq_ids):
    """(group_start int32 [g + 1], shared_blocks int32 [g]) for the sequences in order."""
    ids, ip = _host(seq_ids, np.int64)
    n = len(ids)
    gs = np.zeros(n + 1, np.int32)
    sb = np.zeros(max(n, 1), np.int32)
    ng = _I32()
    _check(lib().kv_shared_prefix_plan(pool, n, ip, gs.ctypes.data_as(C.c_void_p), sb.ctypes.data_as(C.c_void_p),
                                       C.byref(ng)))
    return gs[:ng.value + 1].copy(), sb[:ng.value].copy()


def paged_attention_cascade_workspace_bytes(pool, n_seqs, n_groups, max_group, num_q_heads, max_blocks_per_seq,
                                            opts=None):
    return int(lib().paged_attention_cascade_workspace_bytes(pool, int(n_seqs), int(n_groups), int(max_group),
                                                             int(num_q_heads), int(max_blocks_per_seq),
                                                             C.byref(opts) if opts is not None else None))


def paged_attention_decode_cascade(pool, layer, q, out, block_tables, context_lens, num_q_heads, group_start,
                                   shared_blocks, max_group, opts=None, workspace=None, stream=None):
    """group_start: device int32 [g + 1]; shared_blocks: device int32 [g]."""
    import torch
    _tables(block_tables, context_lens)
    n_seqs, max_blocks = int(block_tables.shape[0]), int(block_tables.shape[1])
    _rows(pool, q, "q", n_seqs, num_q_heads)
    _rows(pool, out, "out", n_seqs, num_q_heads)
    _device_tensor(shared_blocks, "shared_blocks", ndim=1, dtype=torch.int32)
    n_groups = int(shared_blocks.shape[0])
    _device_tensor(group_start, "group_start", dtype=torch.int32, shape=(n_groups + 1,))
    _workspace(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().paged_attention_decode_cascade(pool, int(layer), _dev(q), _dev(out), _dev(block_tables),
                                                _dev(context_lens), n_seqs, max_blocks, int(num_q_heads),
                                                _dev(group_start), _dev(shared_blocks), n_groups, int(max_group),
                                                C.byref(opts) if opts is not None else None, _dev(workspace),
                                                ws_bytes, _stream(stream)))


# -- host tier: swap to pinned host frames -------------------------------------

KV_TIER_HBM, KV_TIER_HOST = 0, 1


def kv_host_frame_bytes(pool):
    return int(lib().kv_host_frame_bytes(pool))


def kv_pool_attach_host(pool, host_frames, n_frames, initial_free_order=None):
    """host_frames: a pinned torch tensor, a raw address, or None (bookkeeping only)."""
    order, ptr = (None, None) if initial_free_order is None else _host(initial_free_order, np.int32)
    hp = host_frames if isinstance(host_frames, int) or host_frames is None else host_frames.data_ptr()
    _check(lib().kv_pool_attach_host(pool, hp, int(n_frames), ptr))
    del order


def _pairs_call(fn, *args, cap):
    out = np.empty((max(cap, 1), 2), np.int32)
    n = _I32()
    _check(fn(*args, out.ctypes.data_as(_P), int(cap), C.byref(n)))
    return out[:n.value].copy()


def kv_seq_swap_out(pool, seq_id, staging, stream=None, cap=1 << 20):
    """(block, frame) pairs [n, 2]."""
    nbytes = 0 if staging is None else staging.numel() * staging.element_size()
    return _pairs_call(lib().kv_seq_swap_out, pool, int(seq_id), _dev(staging), nbytes, _stream(stream), cap=cap)


def kv_seq_swap_in(pool, seq_id, staging, stream=None, cap=1 << 20):
    """(frame, block) pairs [n, 2]."""
    nbytes = 0 if staging is None else staging.numel() * staging.element_size()
    return _pairs_call(lib().kv_seq_swap_in, pool, int(seq_id), _dev(staging), nbytes, _stream(stream), cap=cap)


def kv_seq_swap_out_fenced(pool, seq_id, fence, cap=1 << 20):
    return _pairs_call(lib().kv_seq_swap_out_fenced, pool, int(seq_id), int(fence), cap=cap)


def kv_seq_swap_in_fenced(pool, seq_id, fence, cap=1 << 20):
    return _pairs_call(lib().kv_seq_swap_in_fenced, pool, int(seq_id), int(fence), cap=cap)


def kv_swap_copy(pool, pairs, direction, staging, stream=None):
    arr, ptr = _host(np.asarray(pairs, np.int32).reshape(-1, 2), np.int32)
    nbytes = 0 if staging is None else staging.numel() * staging.element_size()
    _check(lib().kv_swap_copy(pool, ptr, len(arr), int(direction), _dev(staging), nbytes, _stream(stream)))
    del arr


def kv_seq_residency(pool, seq_id, cap=1 << 20):
    """(tiers int32 [n], indices int32 [n]) of the sequence's extended block table."""
    tiers = np.empty(max(cap, 1), np.int32)
    idx = np.empty(max(cap, 1), np.int32)
    n = _I32()
    _check(lib().kv_seq_residency(pool, int(seq_id), int(cap), tiers.ctypes.data_as(_P), idx.ctypes.data_as(_P),
                                  C.byref(n)))
    return tiers[:n.value].copy(), idx[:n.value].copy()


def kv_host_free_list(pool, n_frames):
    out = np.empty(max(n_frames, 1), np.int32)
    n = _I32()
    _check(lib().kv_host_free_list(pool, int(n_frames), out.ctypes.data_as(_P), C.byref(n)))
    return out[:n.value].copy()
