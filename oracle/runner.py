"""Replay a synthetic workload through the oracle (test infrastructure; see oracle/__init__).

Drives :class:`oracle.block_manager.BlockManager` and :class:`oracle.kv_store.KVStore`
with the operations of a :class:`synth.workloads.Workload`.  Per append batch the
block copies requested by copy-on-write are applied first and the new token
rows written afterwards, which is the order in which the copy must precede the
divergent write ([KVM] CoW branching; [BT] §08).  Records every batch's slots
and copy pairs and every decode's block tables and lengths, and evaluates the
float64 attention of any recorded decode.
"""

from __future__ import annotations

import numpy as np

from synth import draws
from synth.draws import TAG_K, TAG_Q, TAG_QCHUNK, TAG_V

from .attention import decode_attention
from .block_manager import BlockManager
from .kv_store import KVStore
from .prefill import chunk_attention
from .quant import QuantKVStore


class OracleReplay:
    def __init__(self, wl, free_order=None, layers=None, writers=None, background=None, eager=False):
        self.wl = wl
        order = draws.free_order(wl.seed, wl.num_blocks) if free_order is None else free_order
        self.bm = BlockManager(wl.num_blocks, wl.block_size, order)
        self.kv_format = getattr(wl, "kv_format", None)
        if self.kv_format:
            if background is not None:
                raise ValueError("a quantised pool has no background pattern")
            self.store = QuantKVStore(wl.num_layers, wl.num_blocks, wl.block_size, wl.num_kv_heads,
                                      wl.head_dim, self.kv_format, wl.dtype, layers)
        else:
            self.store = KVStore(wl.num_layers, wl.num_blocks, wl.block_size, wl.num_kv_heads,
                                 wl.head_dim, draws.storage_np_dtype(wl.dtype), background, layers)
        self.layers = list(range(wl.num_layers)) if layers is None else list(layers)
        self.writers = None if writers is None else set(writers)
        self.appends = []  # (seq_ids, counts, slots, pairs)
        self.decodes = []  # {"seq_ids", "tables", "lengths"}
        self.prefills = []  # {"seq_ids", "counts", "tables", "lengths"} (lengths after the chunk)
        self.swaps = []  # {"kind", "seq", "pairs": [(block, frame)] out / [(frame, block)] in, "length", "positions"}
        # eager: every decode is evaluated when it happens (needed once blocks are reused after a
        # release or a swap-out; otherwise attention() reads the store at the end of the replay)
        self.eager = eager
        self.decode_out = {}  # (decode index, layer) -> [S, Hq, d] float64 (NaN rows for empty sequences)

    def run(self, ops=None):
        for op in (self.wl.ops if ops is None else ops):
            self.apply(op)
        return self

    def gather_f64(self, layer, table, n):
        """K and V [n, Hkv, d] float64 of a sequence: widened stored values, or the
        dequantised values of a quantised pool."""
        if self.kv_format:
            return self.store.gather_f64(layer, table, n)
        kb, vb = self.store.gather(layer, table, n)
        return draws.bits_to_f64(kb, self.wl.dtype), draws.bits_to_f64(vb, self.wl.dtype)

    def rows(self, tag, layer, writer, positions):
        wl = self.wl
        return draws.token_rows(wl.seed, tag, layer, writer, positions, wl.num_kv_heads,
                                wl.head_dim, wl.dtype)

    def apply(self, op):
        kind = op[0]
        if kind == "add":
            self.bm.add(op[1])
        elif kind == "fork":
            self.bm.fork(op[1], op[2])
        elif kind == "release":
            self.bm.release(op[1])
        elif kind == "host":
            sequential = len(op) > 2 and op[2] == "sequential"
            self.bm.attach_host(op[1], None if sequential else draws.host_free_order(self.wl.seed, op[1]))
        elif kind in ("swap_out", "swap_in"):
            seq = op[1]
            if kind == "swap_out":
                pairs = self.bm.swap_out(seq)
                self.store.to_host(pairs)
            else:
                pairs = self.bm.swap_in(seq)
                self.store.from_host(pairs)
            frames = {f: j for j, (tier, f) in enumerate(self.bm.residency(seq)) if tier == "host"} \
                if kind == "swap_out" else None
            self.swaps.append({
                "kind": kind, "seq": seq, "pairs": pairs, "length": self.bm.length(seq),
                # logical block of every pair (table order)
                "positions": [frames[f] for _, f in pairs] if frames is not None else None,
            })
        elif kind in ("append", "prefill"):
            seq_ids, counts = list(op[1]), list(op[2])
            running = {}
            segments = []  # (writer, first position, count)
            for s, c in zip(seq_ids, counts):
                start = running.get(s, self.bm.length(s))
                segments.append((s, start, c))
                running[s] = start + c
            slots, pairs = self.bm.append(seq_ids, counts)
            self.store.copy_blocks(pairs)
            at = 0
            for s, start, c in segments:
                if c and (self.writers is None or s in self.writers):
                    pos = np.arange(start, start + c)
                    for layer in self.layers:
                        self.store.write(layer, slots[at:at + c], self.rows(TAG_K, layer, s, pos),
                                         self.rows(TAG_V, layer, s, pos))
                at += c
            self.appends.append((tuple(seq_ids), tuple(counts), list(slots), list(pairs)))
            if kind == "prefill":
                self.prefills.append({
                    "seq_ids": seq_ids,
                    "counts": counts,
                    "tables": [self.bm.table(s) for s in seq_ids],
                    "lengths": [self.bm.length(s) for s in seq_ids],
                })
        elif kind == "decode":
            seq_ids = list(op[1])
            self.decodes.append({
                "seq_ids": seq_ids,
                "tables": [self.bm.table(s) for s in seq_ids],
                "lengths": [self.bm.length(s) for s in seq_ids],
            })
            if self.eager:
                i = len(self.decodes) - 1
                for layer in self.layers:
                    self.decode_out[(i, layer)] = self._evaluate(i, layer, range(len(seq_ids)))
        else:
            raise ValueError(f"unknown op {kind!r}")

    def query_bits(self, decode_index, layer):
        wl = self.wl
        n = len(self.decodes[decode_index]["seq_ids"])
        return draws.normal_bits(wl.seed, TAG_Q, (decode_index, layer),
                                 (n, wl.num_q_heads, wl.head_dim), wl.dtype)

    def attention(self, decode_index, layer, rows=None, heads=None):
        """float64 outputs [len(rows), Hq, d] of a recorded decode (rows index its batch)."""
        dec = self.decodes[decode_index]
        rows = range(len(dec["seq_ids"])) if rows is None else rows
        if self.eager:
            return self.decode_out[(decode_index, layer)][list(rows)]
        return self._evaluate(decode_index, layer, rows)

    def _evaluate(self, decode_index, layer, rows):
        wl = self.wl
        dec = self.decodes[decode_index]
        q = draws.bits_to_f64(self.query_bits(decode_index, layer), wl.dtype)
        out = []
        for i in rows:
            if dec["lengths"][i] == 0 and self.eager:
                out.append(np.full((wl.num_q_heads, wl.head_dim), np.nan))
                continue
            k, v = self.gather_f64(layer, dec["tables"][i], dec["lengths"][i])
            out.append(decode_attention(q[i], k, v))
        return np.stack(out)

    def prefill_query_bits(self, prefill_index, layer):
        wl = self.wl
        total = sum(self.prefills[prefill_index]["counts"])
        return draws.normal_bits(wl.seed, TAG_QCHUNK, (prefill_index, layer),
                                 (total, wl.num_q_heads, wl.head_dim), wl.dtype)

    def prefill_attention(self, prefill_index, layer, seqs=None, first_rows=None):
        """float64 outputs of a recorded prefill: {batch index: [count, Hq, d]}.

        ``first_rows`` limits each chunk to its first rows; they see no key past
        position h + first_rows - 1, so the keys are cut there too."""
        wl = self.wl
        rec = self.prefills[prefill_index]
        seqs = range(len(rec["seq_ids"])) if seqs is None else seqs
        q = draws.bits_to_f64(self.prefill_query_bits(prefill_index, layer), wl.dtype)
        first = np.concatenate([[0], np.cumsum(rec["counts"])])
        out = {}
        for i in seqs:
            c = rec["counts"][i]
            r = c if first_rows is None else min(c, first_rows)
            n = rec["lengths"][i] - c + r
            k, v = self.gather_f64(layer, rec["tables"][i], n)
            out[i] = chunk_attention(q[first[i]:first[i] + r], k, v)
        return out

    def prefill_rows(self, prefill_index, layer, picks):
        """float64 outputs [len(picks), Hq, d] of single rows (batch index, chunk row) of a
        recorded prefill; row j of a chunk of c tokens is the decode query of position
        length - c + j over the cached positions 0 .. length - c + j."""
        wl = self.wl
        rec = self.prefills[prefill_index]
        q = draws.bits_to_f64(self.prefill_query_bits(prefill_index, layer), wl.dtype)
        first = np.concatenate([[0], np.cumsum(rec["counts"])])
        out = []
        for i, j in picks:
            n = rec["lengths"][i] - rec["counts"][i] + j + 1
            k, v = self.gather_f64(layer, rec["tables"][i], n)
            out.append(decode_attention(q[first[i] + j], k, v))
        return np.stack(out)
