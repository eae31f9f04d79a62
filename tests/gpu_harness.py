"""Replays a synthetic workload through the HIP library (C++ block manager +
device kernels), optionally checking every allocator result against an
oracle replay of the same workload bit for bit.

Used by the GPU tests and by ``__graft_entry__.smoke``.  Inputs come from
:mod:`synth` only; nothing here computes attention.
"""

from __future__ import annotations

import os

import numpy as np
import torch

from pagedattention_decode_amd import binding as B
from pagedattention_decode_amd.pool import PagedKVPool
from synth import draws
from synth.draws import TAG_K, TAG_Q, TAG_QCHUNK, TAG_V


_EXECUTOR = None


def _pool():
    global _EXECUTOR
    if _EXECUTOR is None:
        from concurrent.futures import ThreadPoolExecutor
        _EXECUTOR = ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 4))
    return _EXECUTOR


def to_device_bits(bits: np.ndarray, device="cuda") -> torch.Tensor:
    if bits.dtype == np.uint16:
        return torch.from_numpy(bits.view(np.int16)).to(device)
    return torch.from_numpy(bits.view(np.int32)).to(device)


def bits_to_float_tensor(t: torch.Tensor, dtype: str) -> torch.Tensor:
    return t.view(torch.bfloat16).float() if dtype == draws.BF16 else t.view(torch.float32)


class GpuRun:
    def __init__(self, wl, layers=None, writers=None, opts=None, free_order=None, fill=None,
                 max_blocks=None, ref=None, decode_layers=None, staging_bytes=64 << 20, on_swap=None,
                 decode_steps=None):
        self.wl = wl
        self.layers = list(range(wl.num_layers)) if layers is None else list(layers)
        self.decode_layers = self.layers if decode_layers is None else list(decode_layers)
        # decode ops (by index) whose attention runs; the others only record their tables
        self.decode_steps = None if decode_steps is None else set(decode_steps)
        self.writers = None if writers is None else set(writers)
        self.opts = opts
        self.ref = ref
        order = draws.free_order(wl.seed, wl.num_blocks) if free_order is None else free_order
        self.quantized = bool(getattr(wl, "kv_format", ""))
        self.pool = PagedKVPool(wl.num_layers, wl.num_blocks, wl.block_size, wl.num_kv_heads,
                                wl.head_dim, wl.kv_format or wl.dtype, free_order=order)
        if fill is not None:
            # a known background: every unwritten element (byte, for a quantised pool) holds this pattern
            pattern = fill & 0xFF if self.quantized else fill
            self.pool.raw("k").fill_(pattern)
            self.pool.raw("v").fill_(pattern)
        final = wl.final_lengths()
        longest = max(final.values()) if final else 1
        self.max_blocks = max_blocks or max(1, -(-longest // wl.block_size))
        self.appends = []
        self.decodes = []
        self.decode_outputs = []  # per decode op: {layer: tensor [S, Hq, d] float32}
        self.prefills = []
        self.prefill_outputs = []  # per prefill op: {layer: tensor [sum(counts), Hq, d] float32}
        self.n_append = 0
        self.n_decode = 0
        self.n_prefill = 0
        self.staging_bytes = staging_bytes
        self.on_swap = on_swap  # called as on_swap(run, swap index) after every swap, once its copies are done
        self.swaps = []         # (kind, seq, pairs)

    def rows(self, tag, layer, writer, positions):
        wl = self.wl
        return draws.token_rows(wl.seed, tag, layer, writer, positions, wl.num_kv_heads, wl.head_dim, wl.dtype)

    def run(self, ops=None):
        for op in (self.wl.ops if ops is None else ops):
            self.apply(op)
        torch.cuda.synchronize()
        return self

    def apply(self, op):
        kind = op[0]
        pool = self.pool
        if kind == "add":
            pool.add(op[1])
        elif kind == "fork":
            pool.fork(op[1], op[2])
        elif kind == "release":
            pool.release(op[1])
            # the blocks return once the stream passes the release; waiting here keeps the free
            # list in the oracle's order whatever the timing
            pool.reclaim(True)
        elif kind == "host":
            sequential = len(op) > 2 and op[2] == "sequential"
            pool.attach_host(op[1], None if sequential else draws.host_free_order(self.wl.seed, op[1]),
                             staging_bytes=self.staging_bytes)
        elif kind in ("swap_out", "swap_in"):
            pairs = pool.swap_out(op[1]) if kind == "swap_out" else pool.swap_in(op[1])
            pool.reclaim(True)  # as for release: freed blocks and frames back in the oracle's order
            if self.ref is not None:
                r = self.ref.swaps[len(self.swaps)]
                assert r["kind"] == kind and r["seq"] == op[1]
                assert [tuple(p) for p in pairs.tolist()] == [tuple(p) for p in r["pairs"]], "swap pairs differ"
            self.swaps.append((kind, op[1], pairs))
            if self.on_swap is not None:
                torch.cuda.synchronize()
                self.on_swap(self, len(self.swaps) - 1)
        elif kind == "append":
            seq_ids, counts = list(op[1]), list(op[2])
            segments, running = [], {}
            for s, c in zip(seq_ids, counts):
                start = running.get(s, pool.info(s)[0])
                segments.append((s, start, c))
                running[s] = start + c
            slots, pairs = pool.append(seq_ids, counts)
            if self.ref is not None:
                r_seq, r_cnt, r_slots, r_pairs = self.ref.appends[self.n_append]
                assert list(r_seq) == seq_ids and list(r_cnt) == counts
                assert np.array_equal(slots, np.asarray(r_slots, np.int64)), "slot mapping differs from the oracle"
                assert [tuple(p) for p in pairs.tolist()] == [tuple(p) for p in r_pairs], "CoW pairs differ"
            self.appends.append((slots, pairs))
            self.n_append += 1
            if len(pairs):
                pool.copy(torch.from_numpy(pairs).cuda())
            write_slots = slots.copy()
            at = 0
            keep = []
            for s, start, c in segments:
                if self.writers is not None and s not in self.writers:
                    write_slots[at:at + c] = -1
                else:
                    keep.append((s, start, c, at))
                at += c
            if not keep or len(slots) == 0:
                return
            d_slots = torch.from_numpy(write_slots).cuda()
            # split every kept segment at generator-chunk boundaries and draw in parallel
            tasks = []
            for s, start, c, at in keep:
                pos = start
                while pos < start + c:
                    end = min(start + c, (pos // draws.CHUNK + 1) * draws.CHUNK)
                    tasks.append((s, pos, end - pos, at + pos - start))
                    pos = end
            for layer in self.layers:
                kb = np.zeros((len(slots), self.wl.num_kv_heads, self.wl.head_dim),
                              dtype=draws.storage_np_dtype(self.wl.dtype))
                vb = np.zeros_like(kb)

                def fill(task, layer=layer, kb=kb, vb=vb):
                    s, p0, c, at = task
                    pos = np.arange(p0, p0 + c)
                    kb[at:at + c] = self.rows(TAG_K, layer, s, pos)
                    vb[at:at + c] = self.rows(TAG_V, layer, s, pos)

                if len(tasks) > 4:
                    list(_pool().map(fill, tasks))
                else:
                    for t in tasks:
                        fill(t)
                pool.cache(layer, to_device_bits(kb), to_device_bits(vb), d_slots)
        elif kind == "prefill":
            seq_ids, counts = list(op[1]), list(op[2])
            self.apply(("append", op[1], op[2]))
            tables, lens = pool.tables(seq_ids, self.max_blocks)
            if self.ref is not None:
                rp = self.ref.prefills[self.n_prefill]
                assert rp["seq_ids"] == seq_ids and list(rp["counts"]) == counts
                assert list(lens) == rp["lengths"], "context lengths differ from the oracle"
                for i, t in enumerate(rp["tables"]):
                    assert list(tables[i, :len(t)]) == t, "block table differs from the oracle"
            self.prefills.append({"seq_ids": seq_ids, "counts": counts, "tables": tables, "lengths": lens})
            d_tables = torch.from_numpy(tables).cuda()
            d_lens = torch.from_numpy(lens).cuda()
            d_indptr = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).cuda()
            outs = {}
            for layer in self.decode_layers:
                outs[layer] = self.prefill(self.n_prefill, layer, d_indptr, d_tables, d_lens, max(counts))
            self.prefill_outputs.append(outs)
            self.n_prefill += 1
        elif kind == "decode":
            seq_ids = list(op[1])
            tables, lens = pool.tables(seq_ids, self.max_blocks)
            if self.ref is not None:
                rd = self.ref.decodes[self.n_decode]
                assert rd["seq_ids"] == seq_ids
                assert list(lens) == rd["lengths"], "context lengths differ from the oracle"
                for i, t in enumerate(rd["tables"]):
                    assert list(tables[i, :len(t)]) == t, "block table differs from the oracle"
            self.decodes.append({"seq_ids": seq_ids, "tables": tables, "lengths": lens})
            d_tables = torch.from_numpy(tables).cuda()
            d_lens = torch.from_numpy(lens).cuda()
            outs = {}
            if self.decode_steps is None or self.n_decode in self.decode_steps:
                for layer in self.decode_layers:
                    outs[layer] = self.decode(self.n_decode, layer, d_tables, d_lens, len(seq_ids))
            self.decode_outputs.append(outs)
            self.n_decode += 1
        else:
            raise ValueError(kind)

    def query_bits(self, decode_index, layer, n):
        wl = self.wl
        return draws.normal_bits(wl.seed, TAG_Q, (decode_index, layer), (n, wl.num_q_heads, wl.head_dim), wl.dtype)

    def decode(self, decode_index, layer, d_tables, d_lens, n, opts=None):
        wl = self.wl
        q = to_device_bits(self.query_bits(decode_index, layer, n))
        # outputs and workspace start as all-ones bytes (NaN in both float
        # types): a row the path forgets to write, or a stale partial or
        # counter it reads, shows up in the comparison
        out = torch.empty_like(q)
        out.view(torch.uint8).fill_(0xFF)
        opts = opts if opts is not None else self.opts
        ws_bytes = self.pool.workspace_bytes(n, wl.num_q_heads, d_tables.shape[1], opts)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda") if ws_bytes else None
        if ws is not None:
            ws.fill_(0xFF)
        self.pool.decode(layer, q, out, d_tables, d_lens, wl.num_q_heads, opts, ws)
        return bits_to_float_tensor(out, wl.dtype)


    def prefill_query_bits(self, prefill_index, layer, total):
        wl = self.wl
        return draws.normal_bits(wl.seed, TAG_QCHUNK, (prefill_index, layer), (total, wl.num_q_heads, wl.head_dim),
                                 wl.dtype)

    def prefill(self, prefill_index, layer, d_indptr, d_tables, d_lens, max_q_len, opts=None):
        wl = self.wl
        n = int(d_tables.shape[0])
        total = int(d_indptr[-1].item())
        q = to_device_bits(self.prefill_query_bits(prefill_index, layer, total))
        out = torch.empty_like(q)
        out.view(torch.uint8).fill_(0xFF)  # NaN: rows the path forgets stay visible
        opts = opts if opts is not None else self.opts
        ws_bytes = self.pool.prefill_workspace_bytes(n, total, max_q_len, wl.num_q_heads, d_tables.shape[1], opts)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda") if ws_bytes else None
        if ws is not None:
            ws.fill_(0xFF)
        self.pool.prefill(layer, q, out, d_indptr, d_tables, d_lens, max_q_len, wl.num_q_heads, opts, ws)
        return bits_to_float_tensor(out, wl.dtype)


    def decode_cascade(self, decode_index, layer, opts=None, plan=None, max_group=None, tables=None, lens=None):
        """The recorded decode's queries through paged_attention_decode_cascade, with the
        library's own shared-prefix plan unless one is given."""
        wl = self.wl
        rec = self.decodes[decode_index]
        tables = rec["tables"] if tables is None else tables
        lens = rec["lengths"] if lens is None else lens
        n = len(rec["seq_ids"])
        gs, sb = self.pool.shared_prefix_plan(rec["seq_ids"]) if plan is None else plan
        max_group = int(np.diff(gs).max()) if max_group is None else max_group
        q = to_device_bits(self.query_bits(decode_index, layer, n))
        out = torch.empty_like(q)
        out.view(torch.uint8).fill_(0xFF)
        opts = opts if opts is not None else self.opts
        d_tables = torch.from_numpy(np.ascontiguousarray(tables, dtype=np.int32)).cuda()
        d_lens = torch.from_numpy(np.ascontiguousarray(lens, dtype=np.int32)).cuda()
        d_gs = torch.from_numpy(np.ascontiguousarray(gs, dtype=np.int32)).cuda()
        d_sb = torch.from_numpy(np.ascontiguousarray(sb, dtype=np.int32)).cuda()
        ws_bytes = self.pool.cascade_workspace_bytes(n, len(sb), max_group, wl.num_q_heads, d_tables.shape[1], opts)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
        ws.fill_(0xFF)
        self.pool.decode_cascade(layer, q, out, d_tables, d_lens, wl.num_q_heads, d_gs, d_sb, max_group, opts, ws)
        return bits_to_float_tensor(out, wl.dtype)


def run_workload_on_gpu(wl, **kw):
    return GpuRun(wl, **kw).run()


def attention_errors(got: np.ndarray, expect: np.ndarray):
    """(max abs error, max over rows of the relative L2 error) of [S, Hq, d] outputs."""
    diff = got - expect
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    num = np.sqrt((diff ** 2).sum(axis=-1))
    den = np.sqrt((expect ** 2).sum(axis=-1))
    rel = float((num / np.maximum(den, 1e-30)).max()) if diff.size else 0.0
    return max_abs, rel
