#!/usr/bin/env python3
"""Throughput of the paged decode-attention hot path on one MI355X.

A step is one decode step of the workload through the whole path:
  host:   kv_append_slots (one token per sequence; copy-on-write pairs),
          kv_get_block_tables, upload of slot mapping and tables;
  device: copy_blocks (only when the allocator asked for copies),
          then for every layer reshape_and_cache + paged_attention_decode
          (split-K kernel, then the log-sum-exp merge of split units).
Inputs (queries, new K/V rows) for every timed step are resident in HBM
before the timed region; the pool is filled once, before warm-up.

Workloads (--workload; synthetic, seeded; see synth/workloads.py):
  gqa70b_12x131072       70B-GQA-shaped layer: 12 x 131072 tokens (6.4 GB of
                         KV), Hq=64, Hkv=8, d=128, B=16, bf16, split-K over
                         512-token partitions.   (default: the long-context
                         workload, the largest that fits one GPU)
  qwen3_8b_37x2304       Qwen3-8B-shaped layer: 37 sequences x 2304 tokens,
                         Hq=32, Hkv=8, d=128, B=16, bf16; 4 layer buffers
                         rotated so the 256 MB last-level cache cannot hold
                         the working set (1.4 GB per step).
  shared_prefix_16x8448  16 x 8448 tokens sharing a 6144-token prefix, same
                         shapes, 4 layers.
  agentic_fork_64x33281  64 sequences (4 roots x 16 forks) x ~33K tokens,
                         36 layers.
--cascade (the shared-prefix and fork workloads) decodes through
paged_attention_decode_cascade: the
groups come from kv_shared_prefix_plan every step, each group's shared prefix
is read once; roofline bytes then count the prefix once per group.

--op swap times the host tier: --swap-seqs of the 37 Qwen3-8B-shaped sequences
(36 layers, 2304 tokens, 340 MB of KV each) swapped out to pinned host frames
and back in per step; reported in GB/s over the host link (both directions)
against PCIe Gen5 x16 (64 GB/s per direction).
--op prefill / verify time the multi-query path instead (paged_attention_prefill):
  prefill  the last 512-token chunk of 16 8K-token prompts (7680 cached tokens each),
           reported in TFLOP/s against the bf16 matrix peak;
  verify   8 draft positions for 16 requests with 8184 cached tokens, 4 layers,
           reported in KV GB/s against the HBM peak.

Prints one JSON line (rank 0, one GPU).
"""

import argparse
import gc
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, public specification

# sources whose hash decides whether a committed counter summary still describes
# the kernels: the kernel file and the headers its device code includes
DECODE_SOURCES = ("kernels.hip", "device_common.h", "pool_internal.h")
CASCADE_SOURCES = ("cascade.hip", "device_common.h", "pool_internal.h")
PREFILL_SOURCES = ("prefill.hip", "device_common.h", "pool_internal.h")
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, public specification


class no_gc:
    """Python's cyclic garbage collector paused for a timed region (a full
    collection over torch's object graph takes tens of milliseconds and would
    land inside some step at random); one collection runs just before."""

    def __enter__(self):
        gc.collect()
        gc.disable()

    def __exit__(self, *exc):
        gc.enable()


# GPU cycles of the spin kernel that gives the host a head start before the
# attention calls are timed one by one
HEAD_START_CYCLES = 2_000_000


def time_calls(torch, B, stream, n, call, **opt_kwargs):
    """Per-call timing of n attention calls, call(j, opts) for j < n, issued
    back to back behind a short GPU spin so that the host is ahead and no call
    waits for its own enqueue.  Each call carries kv_timing_events, which the
    library attaches to its own kernel launches: start .. kernel_stop is the
    kernel streaming the K/V cache, start .. stop the whole call.  Returns
    (kernel ms, call ms) per call."""
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(n)]
    for t in evs:
        for e in t:
            e.record(stream)  # gives each its HIP event
    opts = [B.attention_options(timing=t, **opt_kwargs) for t in evs]
    torch.cuda.synchronize()
    with no_gc():
        torch.cuda._sleep(HEAD_START_CYCLES)
        for j in range(n):
            call(j, opts[j])
        torch.cuda.synchronize()
    return [s.elapsed_time(k) for s, k, _ in evs], [s.elapsed_time(e) for s, _, e in evs]


def pcts(ms):
    import numpy as np
    return [round(float(np.percentile(ms, q)) * 1e3, 2) for q in (10, 50, 90)]


# layer buffers per step of each decode workload
DECODE_LAYERS = {"qwen3_8b_37x2304": 4, "shared_prefix_16x8448": 4, "gqa70b_12x131072": 1,
                 "agentic_fork_64x33281": 36}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0,
                    help="timed steps (0 = 100 for the decode workloads, 20 for the fork workload and the other ops)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gqa70b_12x131072", choices=list(DECODE_LAYERS),
                    help="the decode workload of --op decode")
    ap.add_argument("--kv", default="bf16", choices=["bf16", "q8_0", "q4_0"],
                    help="storage of the KV pool (decode, prefill, verify): bf16, or q8_0 / q4_0 codes with one 2-byte "
                         "scale per 32 values (written by reshape_and_cache, dequantised in the kernel)")
    ap.add_argument("--block-size", type=int, default=0,
                    help="tokens per block of the pool (0 = the workload's, 16); decode reads bf16 pools of block "
                         "size 4, 8, 32 and 64 with the matrix-core kernel too, --op prefill / verify with the "
                         "multi-query kernels")
    ap.add_argument("--swap-seqs", type=int, default=8, help="--op swap: sequences swapped out and back in per step")
    ap.add_argument("--op", default="decode", choices=["decode", "prefill", "verify", "swap"],
                    help="decode: the decode step of --workload; prefill: the last 512-token chunk of 16 "
                         "8K prompts; verify: 8 draft positions for 16 requests with 8K contexts")
    ap.add_argument("--cascade", action="store_true",
                    help="decode through paged_attention_decode_cascade (shared prefixes read once per group)")
    ap.add_argument("--layers", type=int, default=0, help="layer buffers (0 = workload default)")
    ap.add_argument("--partition", type=int, default=-1, help="partition tokens (-1 = workload default)")
    ap.add_argument("--kernel", default="auto", choices=["auto", "mfma", "generic", "mfma_staged_table", "valu"],
                    help="mfma_staged_table: the matrix-core kernel with each wave's block-table entries staged in "
                         "LDS (bf16, B = 16), for comparison with the scalar table reads of mfma; valu: the same "
                         "split-K kernel with vector-ALU dot products instead of matrix instructions (bf16, B = 16, "
                         "d = 128, G = 4 or 8)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--seed", type=int, default=0, help="0 = the workload's seed")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 5 device-to-device copies of MIB MiB (a plain copy of known size, used to "
                         "calibrate the FETCH_SIZE / WRITE_SIZE counters) and exit")
    g = ap.add_argument_group("summaries of rocprofv3 output for profiles/ (no GPU needed)")
    g.add_argument("--summarize-trace", metavar="DIR", help="a --kernel-trace --stats output directory")
    g.add_argument("--summarize-counters", metavar="DIR",
                   help="directory with pmc_<name>_FETCH_SIZE/, pmc_<name>_WRITE_SIZE/, pmc_cal_FETCH_SIZE/, "
                        "pmc_cal_WRITE_SIZE/ and their .log files")
    g.add_argument("--summarize-activity", metavar="DIR",
                   help="directory with act_<kind>_1/ and act_<kind>_2/ (vector-ALU and matrix-core activity "
                        "counters of one workload per KV storage kind) and their .log files")
    g.add_argument("--summary-kinds", default="bf16,q8_0,q4_0", help="--summarize-activity: the storage kinds")
    g.add_argument("--summary-name", default="", help="<name> of the pmc_<name>_* runs")
    g.add_argument("--summary-workload", default="", help="workload name of hbm_traffic_<workload>.json")
    g.add_argument("--summary-kernels", default="attn_mfma_kernel,merge_sk_kernel",
                   help="kernels of one call, the one streaming the cache first")
    g.add_argument("--summary-sources", default=",".join(DECODE_SOURCES),
                   help="csrc files whose hash the summary records")
    g.add_argument("--summary-file", default="", help="markdown file name in profiles/ (without .md)")
    g.add_argument("--summary-title", default="")
    g.add_argument("--summary-command", default="", help="bench.py arguments of the profiled run")
    return ap.parse_args()


def copy_calibration(mib):
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_copy": n, "copies": 5}), flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.summarize_counters:
        summarize_counters(args)
        return
    if args.summarize_trace:
        summarize_trace(args)
        return
    if args.summarize_activity:
        summarize_activity(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU form)", file=sys.stderr)
        sys.exit(2)
    if args.steps <= 0:
        # a decode step is ~0.35 ms (37 x 2304, 4 layers) to ~1.1 ms (12 x 131072): 100 of them
        # keep the timed region long against the host's occasional stalls of a few milliseconds
        args.steps = 100 if args.op == "decode" and args.workload != "agentic_fork_64x33281" else 20

    if args.op == "swap":
        swap_bench(args)
        return
    if args.op != "decode":
        multi_query_bench(args)
        return

    import numpy as np
    import torch

    from pagedattention_decode_amd import binding as B
    from pagedattention_decode_amd.pool import PagedKVPool
    from synth import draws, workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    fork = args.workload == "agentic_fork_64x33281"
    base = workloads.agentic_fork(steps=1) if fork else workloads.get_workload(args.workload)
    if args.block_size and args.block_size != base.block_size:
        from dataclasses import replace
        # the same tokens in blocks of another size (plus one partly filled block per sequence)
        n_dec = len(next(op for op in base.ops if op[0] == "decode")[1])
        base = replace(base, block_size=args.block_size,
                       num_blocks=-(-base.num_blocks * base.block_size // args.block_size) + n_dec)
    L = args.layers or DECODE_LAYERS[args.workload]
    seed = args.seed or base.seed
    partition = base.partition_tokens if args.partition < 0 else args.partition
    kernel = {"auto": B.KV_KERNEL_AUTO, "mfma": B.KV_KERNEL_MFMA, "generic": B.KV_KERNEL_GENERIC,
              "mfma_staged_table": B.KV_KERNEL_MFMA_STAGED_TABLE, "valu": B.KV_KERNEL_VALU}[args.kernel]
    opts = B.attention_options(partition_tokens=partition, kernel=kernel)
    Hq, Hkv, d, Bs = base.num_q_heads, base.num_kv_heads, base.head_dim, base.block_size

    # setup = everything before the per-step ops; a step appends one token per
    # decoding sequence when the workload does so, then decodes
    ops = base.ops
    first_step = next(i for i, op in enumerate(ops)
                      if op[0] == "decode" or (op[0] == "append" and set(op[2]) == {1}))
    setup_ops = ops[:first_step]
    step_ops = ops[first_step:]
    decode_seqs = list(next(op for op in step_ops if op[0] == "decode")[1])
    step_appends = any(op[0] == "append" for op in step_ops)
    S = len(decode_seqs)

    total_steps = args.warmup + args.steps
    # room for the tokens the steps append (and one copy-on-write block per sequence) on top of
    # the workload's pool; the per-step work does not depend on the pool's size
    num_blocks = base.num_blocks + (S * (-(-total_steps // Bs) + 2) if step_appends else 0)
    pool = PagedKVPool(L, num_blocks, Bs, Hkv, d, args.kv, free_order=draws.free_order(seed, num_blocks))
    # bytes of one token's K and V in one layer, as stored (codes + scales when quantised)
    kv_tok = 2 * Hkv * (d * 2 if args.kv == "bf16" else d * (8 if args.kv == "q8_0" else 4) // 8 + d // 32 * 2)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)

    def randn_bf16(*shape):
        return torch.randn(shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)

    # ---- fill the pool (untimed) -----------------------------------------
    t_fill = time.time()
    for op in setup_ops:
        if op[0] == "add":
            pool.add(op[1])
        elif op[0] == "fork":
            pool.fork(op[1], op[2])
        elif op[0] == "append":
            slots, pairs = pool.append(op[1], op[2])
            assert len(pairs) == 0
            chunk = 1 << 17
            for at in range(0, len(slots), chunk):
                d_slots = torch.from_numpy(slots[at:at + chunk]).to(dev)
                n = d_slots.numel()
                for layer in range(L):
                    pool.cache(layer, randn_bf16(n, Hkv, d), randn_bf16(n, Hkv, d), d_slots)
    torch.cuda.synchronize()
    t_fill = time.time() - t_fill

    lens0 = np.array([pool.info(s)[0] for s in decode_seqs])
    max_blocks = int(math.ceil((lens0.max() + (total_steps if step_appends else 0)) / Bs)) + 1
    # every step's inputs, resident in HBM before the timed region: per layer the queries and,
    # when the workload appends, the new K and V rows; one flat buffer per step
    n_q, n_kv = S * Hq * d, (S * Hkv * d if step_appends else 0)
    per_layer = n_q + 2 * n_kv
    inputs = randn_bf16(total_steps, L * per_layer)

    def layer_inputs(buf, layer):
        at = layer * per_layer
        q = buf[at:at + n_q].view(S, Hq, d)
        if not n_kv:
            return q, None, None
        k = buf[at + n_q:at + n_q + n_kv].view(S, Hkv, d)
        v = buf[at + n_q + n_kv:at + per_layer].view(S, Hkv, d)
        return q, k, v

    out = torch.empty((S, Hq, d), dtype=torch.bfloat16, device=dev)
    if args.cascade:
        # max_group sizes the prefix grid: the largest group of the first step's plan (the fork
        # structure does not change while the sequences decode); the workspace covers any number
        # of groups, since the prefix partition depends on it
        gs0, _ = pool.shared_prefix_plan(np.asarray(decode_seqs, np.int64))
        max_group = int(np.diff(gs0).max())
        ws_bytes = max(pool.cascade_workspace_bytes(S, ng, max_group, Hq, max_blocks, opts)
                       for ng in range(1, S + 1))
    else:
        ws_bytes = pool.workspace_bytes(S, Hq, max_blocks, opts)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    # the step's host data: slot mapping (int64), tables, lengths and the cascade plan (int32)
    # packed in one pinned buffer; a step sends what changed since the last upload
    off_t = 8 * S
    off_l = off_t + 4 * S * max_blocks
    off_p = off_l + 4 * S
    up_bytes = off_p + 4 * (2 * S + 1)
    d_up = torch.empty((up_bytes,), dtype=torch.uint8, device=dev)
    d_slots = d_up[:off_t].view(torch.int64)
    d_tables = d_up[off_t:off_l].view(torch.int32).view(S, max_blocks)
    d_lens = d_up[off_l:off_p].view(torch.int32)
    d_plan = d_up[off_p:].view(torch.int32)
    # pinned upload buffers in flight: the host may run this many steps ahead of the device, so
    # that a stall of a few milliseconds on the host leaves the device's queue non-empty
    ring = 32
    h_up = [torch.empty((up_bytes,), dtype=torch.uint8).pin_memory() for _ in range(ring)]
    h_np = [h.numpy() for h in h_up]
    h_slots = [h[:off_t].view(np.int64) for h in h_np]
    h_tables = [h[off_t:off_l].view(np.int32).reshape(S, max_blocks) for h in h_np]
    h_lens = [h[off_l:off_p].view(np.int32) for h in h_np]
    h_plan = [h[off_p:].view(np.int32) for h in h_np]
    ring_ev = [None] * ring
    seq_arr = np.asarray(decode_seqs, np.int64)
    # what the device holds from the previous upload: only the parts that changed are sent
    # (the block tables change when a sequence crosses a block or copies on write; the slot
    # mapping and the lengths with every appended token)
    dev_tables = [None]
    dev_tail = [None]
    stream = torch.cuda.current_stream()

    logical_bytes = [0]
    first_tables = []  # the first timed step's tables and lengths (for its unique bytes)
    n_copies = [0]
    n_groups = [0]
    read_bytes = [0]  # KV bytes the path reads (shared prefixes once per group with --cascade)

    def attention(layer, q, o):
        if args.cascade:
            ng = n_groups[0]
            pool.decode_cascade(layer, q, out, d_tables, d_lens, Hq, d_plan[:ng + 1], d_plan[ng + 1:2 * ng + 1],
                                max_group, o, ws)
        else:
            pool.decode(layer, q, out, d_tables, d_lens, Hq, o, ws)

    def layers(buf):
        for layer in range(L):
            q, k, v = layer_inputs(buf, layer)
            if step_appends:
                pool.cache(layer, k, v, d_slots)
            attention(layer, q, opts)

    def step(i, timed):
        slot = i % ring
        if ring_ev[slot] is not None:
            ring_ev[slot].synchronize()
        pairs = np.zeros((0, 2), np.int64)
        if step_appends:
            slots, pairs = pool.append(seq_arr, None)
            h_slots[slot][:] = slots
        tables, lens = B.kv_get_block_tables(pool.handle, seq_arr, max_blocks)
        h_tables[slot][:] = tables
        h_lens[slot][:] = lens
        if args.cascade:
            gs, sb = pool.shared_prefix_plan(seq_arr)
            ng = len(sb)
            assert int(np.diff(gs).max()) <= max_group, "a fork group outgrew the first step's plan"
            h_plan[slot][:ng + 1] = gs
            h_plan[slot][ng + 1:2 * ng + 1] = sb
            n_groups[0] = ng
            # tokens the cascade reads: each group's shared prefix once, every member's suffix
            shared_tok = np.repeat(sb.astype(np.int64) * Bs, np.diff(gs))
            read_tokens = int(sb.astype(np.int64).sum()) * Bs + int((lens.astype(np.int64) - shared_tok).sum())
        else:
            read_tokens = int(lens.astype(np.int64).sum())
        if dev_tables[0] is None or not np.array_equal(h_tables[slot], dev_tables[0]):
            d_up.copy_(h_up[slot], non_blocking=True)
            dev_tables[0] = h_tables[slot].copy()
            dev_tail[0] = h_np[slot][off_l:].copy()
        else:
            if step_appends:
                d_up[:off_t].copy_(h_up[slot][:off_t], non_blocking=True)
            if not np.array_equal(h_np[slot][off_l:], dev_tail[0]):
                d_up[off_l:].copy_(h_up[slot][off_l:], non_blocking=True)
                dev_tail[0] = h_np[slot][off_l:].copy()
        ev = torch.cuda.Event()
        ev.record(stream)
        ring_ev[slot] = ev
        if len(pairs):
            pool.copy(torch.from_numpy(pairs).to(dev, non_blocking=False))
            n_copies[0] += len(pairs)
        layers(inputs[i])
        if timed:
            logical_bytes[0] += L * int(lens.astype(np.int64).sum()) * kv_tok
            read_bytes[0] += L * read_tokens * kv_tok
            if not first_tables:
                first_tables.append((tables.copy(), lens.copy()))
        return lens

    for i in range(args.warmup):
        step(i, False)
    lens_hist = []
    with no_gc():
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.warmup, total_steps):
            lens_hist.append(step(i, True))
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    wall = t1 - t0
    ms_step = wall / args.steps * 1e3

    attn_name = "paged_attention_decode_cascade" if args.cascade else "paged_attention_decode"
    # the timed steps' attention calls once more, each timed on its own (the
    # tables and lengths of the last step, layers in turn)
    kern_ms, attn_ms = time_calls(torch, B, stream, args.steps * L,
                                  lambda j, o: attention(j % L, layer_inputs(inputs[args.warmup + j // L], j % L)[0], o),
                                  partition_tokens=partition, kernel=kernel)
    attn_avg_s = float(np.mean(attn_ms)) / 1e3
    kern_avg_s = float(np.mean(kern_ms)) / 1e3
    n_launch = args.steps * L
    blocks_per_launch = float(np.mean([np.ceil(l / Bs).sum() for l in lens_hist]))
    qo_tab = 2 * S * Hq * d * 2 + 4 * blocks_per_launch  # queries, outputs, table entries
    # KV bytes a launch must read at least: every physical block once, as far as the longest
    # context reading it reaches (sharing sequences read a shared block once between them);
    # the contexts grow by one token per step, so the mean of the first and last timed steps
    last_tables = B.kv_get_block_tables(pool.handle, seq_arr, max_blocks)
    unique_kv_bytes = 0.5 * (unique_tokens(*first_tables[0], Bs) + unique_tokens(*last_tables, Bs)) * kv_tok
    logical_per_launch = logical_bytes[0] / n_launch + qo_tab
    # the cascade reads each group's shared prefix once (read_bytes), the plain decode is held to
    # the unique bytes; without sharing both equal the logical bytes
    ideal_per_launch = (read_bytes[0] / n_launch if args.cascade else unique_kv_bytes) + qo_tab
    # the roofline is that of the kernel streaming the cache (the split-K
    # partition kernel); the cascade's bytes are only defined for the whole call
    roof_s = attn_avg_s if args.cascade else kern_avg_s
    achieved = ideal_per_launch / roof_s / 1e9
    value = logical_bytes[0] / wall / 1e9
    tok_per_s_layer = S * L * args.steps / wall

    traffic_key = (base.name + ("" if args.kv == "bf16" else f"_{args.kv}") + ("_cascade" if args.cascade else "") +
                   ("" if Bs == 16 else f"_b{Bs}"),
                   CASCADE_SOURCES if args.cascade else DECODE_SOURCES,
                   "traffic_bytes_per_call" if args.cascade else "traffic_bytes_per_launch")
    result = {
        "metric": "paged-decode KV GB/s (% of HBM peak) + attention tokens/s per layer",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": base.name,
            "description": base.description,
            "layers_per_step": L,
            "sequences": S,
            "context_tokens_first_step": int(lens_hist[0].max()) if lens_hist else None,
            "partition_tokens": partition or "auto",
            "kernel": args.kernel,
            "kv_storage": args.kv,
            "block_size": Bs,
            "kv_bytes_per_token_per_layer": kv_tok,
            "pool_blocks": num_blocks,
            "step": (f"append + {L} x (reshape_and_cache + {attn_name})" if step_appends
                     else f"{L} x {attn_name}"),
        },
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "attn_tokens_per_s_per_layer": round(tok_per_s_layer, 1),
        "attn_call_tokens_per_s_per_layer": round(S / attn_avg_s, 1),
        "attn_call_us": round(attn_avg_s * 1e6, 2),
        "attn_call_us_p10_p50_p90": pcts(attn_ms),
        "attn_kernel_us": round(kern_avg_s * 1e6, 2),
        "attn_kernel_us_p10_p50_p90": pcts(kern_ms),
        "call_achieved_gbs": round(ideal_per_launch / attn_avg_s / 1e9, 1),
        "call_frac": round(ideal_per_launch / attn_avg_s / 1e9 / HBM_PEAK_GBS, 4),
        "unique_kv_bytes_per_launch": int(unique_kv_bytes),
        # logical bytes (every sequence's context through its own table) over the kernel's time:
        # above the HBM peak where sequences share blocks that the caches serve
        "logical_achieved_gbs": round(logical_per_launch / roof_s / 1e9, 1),
        "cow_copies": n_copies[0],
        "fill_seconds": round(t_fill, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(*traffic_key),
            "kernel": ("paged_attention_decode_cascade (whole call: attn_cascade_kernel over the prefix and "
                       "suffix units, then cascade_merge_kernel)" if args.cascade
                       else "attn_mfma_kernel (split-K partition kernel)"),
            "duration_us": round(roof_s * 1e6, 2),
            "algorithmic_bytes_per_launch": int(ideal_per_launch),
            "algorithmic_bytes": ("each group's shared prefix once, every member's own blocks, q, out, table "
                                  "entries" if args.cascade else
                                  "every physical block read once (as far as the longest context reading it "
                                  "reaches), q, out, table entries"),
        },
        "cpu_baseline": None,
    }
    ratio = traffic_ratio(*traffic_key)
    if ratio:
        # HBM bytes the counters saw against the algorithmic bytes of the same run, and the HBM
        # rate that ratio gives over this run's bytes and measured duration
        result["roofline"]["traffic_over_algorithmic"] = round(ratio, 4)
        result["roofline"]["traffic_gbs"] = round(ratio * ideal_per_launch / roof_s / 1e9, 1)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args)
    print(json.dumps(result), flush=True)


def unique_tokens(tables, lens, block_size):
    """Tokens of the distinct physical blocks the batch reads: each block counted
    once, with the most slots any of its readers sees."""
    import numpy as np
    lens = np.asarray(lens, np.int64)
    nb = -(-lens // block_size)
    j = np.arange(tables.shape[1])[None, :]
    live = j < nb[:, None]
    valid = np.minimum(block_size, lens[:, None] - j * block_size)
    blocks, valid = tables[live].astype(np.int64), valid[live]
    if blocks.size == 0:
        return 0
    best = np.zeros(int(blocks.max()) + 1, np.int64)
    np.maximum.at(best, blocks, valid)
    return int(best.sum())


def multi_query_bench(args):
    """Chunked prefill or draft verification through paged_attention_prefill.

    A step is, for every layer, reshape_and_cache of the chunk's K/V rows (into
    the slots the chunk owns) followed by the multi-query attention of the
    chunk's queries.  The history is written once before warm-up; queries and
    chunk rows for every timed step are resident in HBM.
    """
    import numpy as np
    import torch

    from pagedattention_decode_amd import binding as B
    from pagedattention_decode_amd.pool import PagedKVPool
    from synth import draws, workloads

    from dataclasses import replace

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    prefill = args.op == "prefill"
    base = workloads.prefill_last_chunk() if prefill else workloads.verify_drafts()
    if args.block_size and args.block_size != base.block_size:
        # the same tokens in blocks of another size (plus one partly filled block per sequence)
        n_seq = len(next(op for op in base.ops if op[0] == "prefill")[1])
        base = replace(base, block_size=args.block_size,
                       num_blocks=-(-base.num_blocks * base.block_size // args.block_size) + n_seq)
    L = args.layers or (1 if prefill else 4)
    seed = args.seed or base.seed
    Hq, Hkv, d, Bs = base.num_q_heads, base.num_kv_heads, base.head_dim, base.block_size
    hist_op = next(op for op in base.ops if op[0] == "append")
    chunk_op = next(op for op in base.ops if op[0] == "prefill")
    seqs, hist, counts = list(chunk_op[1]), list(hist_op[2]), list(chunk_op[2])
    S, c = len(seqs), counts[0]
    opts = B.attention_options(partition_tokens=max(args.partition, 0))

    pool = PagedKVPool(L, base.num_blocks, Bs, Hkv, d, args.kv, free_order=draws.free_order(seed, base.num_blocks))
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)

    def randn_bf16(*shape):
        return torch.randn(shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)

    t_fill = time.time()
    for s in seqs:
        pool.add(s)
    slots, _ = pool.append(seqs, hist)
    d_hist = torch.from_numpy(slots).to(dev)
    for layer in range(L):
        pool.cache(layer, randn_bf16(len(slots), Hkv, d), randn_bf16(len(slots), Hkv, d), d_hist)
    chunk_slots, _ = pool.append(seqs, counts)
    d_slots = torch.from_numpy(chunk_slots).to(dev)
    torch.cuda.synchronize()
    t_fill = time.time() - t_fill

    total_q = S * c
    max_blocks = int(math.ceil((max(hist) + c) / Bs))
    tables, lens = B.kv_get_block_tables(pool.handle, np.asarray(seqs, np.int64), max_blocks)
    d_tables = torch.from_numpy(tables).to(dev)
    d_lens = torch.from_numpy(lens).to(dev)
    d_indptr = torch.arange(0, total_q + 1, c, dtype=torch.int32, device=dev)
    total_steps = args.warmup + args.steps
    q_in = [[randn_bf16(total_q, Hq, d) for _ in range(L)] for _ in range(total_steps)]
    kv_in = [[(randn_bf16(total_q, Hkv, d), randn_bf16(total_q, Hkv, d)) for _ in range(L)]
             for _ in range(total_steps)]
    out = torch.empty((total_q, Hq, d), dtype=torch.bfloat16, device=dev)
    ws_bytes = pool.prefill_workspace_bytes(S, total_q, c, Hq, max_blocks, opts)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(i, timed):
        for layer in range(L):
            k_new, v_new = kv_in[i][layer]
            pool.cache(layer, k_new, v_new, d_slots)
            pool.prefill(layer, q_in[i][layer], out, d_indptr, d_tables, d_lens, c, Hq, opts, ws)

    for i in range(args.warmup):
        step(i, False)
    with no_gc():
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.warmup, total_steps):
            step(i, True)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    kern_ms, attn_ms = time_calls(
        torch, B, stream, args.steps * L,
        lambda j, o: pool.prefill(j % L, q_in[args.warmup + j // L][j % L], out, d_indptr, d_tables, d_lens, c, Hq,
                                  o, ws),
        partition_tokens=max(args.partition, 0))
    attn_s = float(np.mean(attn_ms)) / 1e3
    kern_s = float(np.mean(kern_ms)) / 1e3
    n = lens.astype(np.int64)
    pairs = int(sum(c * (int(x) - c) + c * (c + 1) // 2 for x in n))  # query-key pairs per head
    flops = 4 * d * Hq * pairs                                          # QK^T and PV, per layer call
    # each sequence's keys and values as stored (codes and scales for a quantised pool)
    kv_per_tok = 2 * Hkv * (d * 2 if args.kv == "bf16" else d * (8 if args.kv == "q8_0" else 4) // 8 + d // 16)
    kv_bytes = int(n.sum()) * kv_per_tok
    quant = args.kv != "bf16"  # raw tiles: the multi-query kernel for quantised pools
    ideal_bytes = kv_bytes + 2 * total_q * Hq * d * 2 + 4 * int(np.ceil(n / Bs).sum())
    calls = args.steps * L
    result = {
        "metric": ("multi-query paged attention TFLOP/s (chunked prefill)" if prefill
                   else "paged-verification KV GB/s (% of HBM peak)"),
        "value": round(flops * calls / wall / 1e12, 2) if prefill else round(kv_bytes * calls / wall / 1e9, 2),
        "unit": "TFLOP/s" if prefill else "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": base.name,
            "description": base.description,
            "layers_per_step": L,
            "sequences": S,
            "chunk_tokens": c,
            "history_tokens": int(hist[0]),
            "partition_tokens": args.partition if args.partition > 0 else "auto",
            "kv_storage": args.kv,
            "kv_bytes_per_token_per_layer": kv_per_tok,
            "block_size": Bs,
            "step": f"{L} x (reshape_and_cache of the chunk + paged_attention_prefill)",
        },
        "attn_call_us": round(attn_s * 1e6, 2),
        "attn_call_us_p10_p50_p90": pcts(attn_ms),
        "attn_kernel_us": round(kern_s * 1e6, 2),
        "attn_kernel_us_p10_p50_p90": pcts(kern_ms),
        "chunk_tokens_per_s_per_layer": round(total_q / attn_s, 1),
        "query_key_pairs_per_head": pairs,
        "fill_seconds": round(t_fill, 2),
        "roofline": ({
            "bound": "mfma",
            "achieved": round(flops / kern_s / 1e12, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(flops / kern_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": None if quant else measured_traffic(base.name, PREFILL_SOURCES),
            "kernel": ("attn_prefill_q_kernel (multi-query kernel, quantised tiles)" if quant
                       else "attn_prefill_lds_kernel (multi-query kernel)"),
            "duration_us": round(kern_s * 1e6, 2),
            "algorithmic_flops_per_launch": flops,
        } if prefill else {
            "bound": "hbm",
            "achieved": round(ideal_bytes / kern_s / 1e9, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(ideal_bytes / kern_s / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": None if quant else measured_traffic(base.name, PREFILL_SOURCES),
            "kernel": ("attn_prefill_q_kernel (multi-query kernel, quantised tiles)" if quant
                       else "attn_prefill_lds_kernel (multi-query kernel)"),
            "duration_us": round(kern_s * 1e6, 2),
            "algorithmic_bytes_per_launch": ideal_bytes,
        }),
        "call_frac": round((flops / attn_s / 1e12 / MFMA_BF16_PEAK_TFLOPS) if prefill
                           else (ideal_bytes / attn_s / 1e9 / HBM_PEAK_GBS), 4),
        "cpu_baseline": None if args.no_cpu_baseline else multi_query_cpu_baseline(
            args, base if args.kv == "bf16" else replace(base, kv_format=args.kv)),
    }
    print(json.dumps(result), flush=True)


def multi_query_cpu_baseline(args, wl):
    """The fp64 oracle's chunk attention of sequence 0 of the workload, repeated."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle.runner import OracleReplay

    cores = len(os.sched_getaffinity(0))
    ref = OracleReplay(wl, writers={0}).run()
    rec = ref.prefills[0]
    # the first rows of sequence 0's chunk (all of a verification chunk)
    rows = min(rec["counts"][0], 32)
    c, n = rows, rec["lengths"][0] - rec["counts"][0] + rows
    pairs = c * (n - c) + c * (c + 1) // 2
    flops = 4 * wl.head_dim * wl.num_q_heads * pairs
    kv_bytes = n * 2 * wl.num_kv_heads * wl.head_dim * wl.elem_bytes
    reps = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=cores):
        while True:
            ref.prefill_attention(0, 0, seqs=[0], first_rows=rows)
            reps += 1
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
    wall = time.perf_counter() - t0
    prefill = args.op == "prefill"
    return {
        "value": round(flops * reps / wall / 1e12, 6) if prefill else round(kv_bytes * reps / wall / 1e9, 4),
        "unit": "TFLOP/s" if prefill else "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"the oracle's chunk attention of the first {c} queries of sequence 0's chunk "
                  f"(keys 0..{n - 1}), repeated {reps} times in {wall:.1f} s",
        "chunk_tokens_per_s_per_layer": round(c * reps / wall, 3),
    }


PCIE_GEN5_X16_GBS = 64.0  # per direction, public specification of the MI355X host link


def swap_bench(args):
    """Swap round trips over the host link ([KVM] asynchronous paged swap).

    A step swaps --swap-seqs sequences out (kv_seq_swap_out, one call each,
    all on one stream) and then back in (kv_seq_swap_in).  The pool is the
    Qwen3-8B-shaped workload with all 36 layers, so a frame is one block of
    every layer (16 x 147456 bytes).  HIP events time each direction on the
    stream; a plain pinned hipMemcpy of the same bytes is timed beside it as
    the link's practical ceiling.
    """
    import numpy as np
    import torch

    from pagedattention_decode_amd.pool import PagedKVPool
    from synth import draws, workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = workloads.qwen_independent()
    L = args.layers or 36
    seed = args.seed or wl.seed
    Hkv, d, Bs = wl.num_kv_heads, wl.head_dim, wl.block_size
    # headroom of two swap sets: a swap-in takes fresh blocks while the last swap-out's
    # blocks may still wait for their copies to finish
    n_blocks = wl.num_blocks + 2 * args.swap_seqs * 144
    pool = PagedKVPool(L, n_blocks, Bs, Hkv, d, args.kv, free_order=draws.free_order(seed, n_blocks))
    seqs = list(range(37))
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    t_fill = time.time()
    for s_ in seqs:
        pool.add(s_)
    slots, _ = pool.append(seqs, [2304] * len(seqs))
    d_slots = torch.from_numpy(slots).to(dev)
    for layer in range(L):
        k = torch.randn((len(slots), Hkv, d), generator=gen, device=dev).to(torch.bfloat16)
        v = torch.randn((len(slots), Hkv, d), generator=gen, device=dev).to(torch.bfloat16)
        pool.cache(layer, k, v, d_slots)
    torch.cuda.synchronize()
    t_fill = time.time() - t_fill
    moved = seqs[:args.swap_seqs]
    blocks = sum(pool.info(s_)[1] for s_ in moved)
    pool.attach_host(2 * blocks + 16, staging_bytes=64 << 20)  # headroom as for the blocks
    F = pool.frame_bytes
    nbytes = blocks * F
    stream = torch.cuda.current_stream()

    def step(timed):
        # the previous step's freed blocks and frames come back once its copies are done
        # (a host wait: the host runs at most one step ahead of the copies)
        pool.reclaim(True)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        for s_ in moved:
            pool.swap_out(s_)
        e[1].record(stream)
        for s_ in moved:
            pool.swap_in(s_)
        e[2].record(stream)
        return e

    for _ in range(args.warmup):
        step(False)
    with no_gc():
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        evs = [step(True) for _ in range(args.steps)]
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    out_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    in_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    pool.check()

    # the link's practical ceiling: one plain pinned copy of the same bytes each way
    host = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    devbuf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    for _ in range(2):
        host.copy_(devbuf, non_blocking=True)
        devbuf.copy_(host, non_blocking=True)
    torch.cuda.synchronize()
    c = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    c[0].record(stream)
    host.copy_(devbuf, non_blocking=True)
    c[1].record(stream)
    devbuf.copy_(host, non_blocking=True)
    c[2].record(stream)
    torch.cuda.synchronize()
    plain_out = nbytes / (c[0].elapsed_time(c[1]) / 1e3) / 1e9
    plain_in = nbytes / (c[1].elapsed_time(c[2]) / 1e3) / 1e9

    gbs_out = nbytes / (out_ms / 1e3) / 1e9
    gbs_in = nbytes / (in_ms / 1e3) / 1e9
    value = 2 * nbytes * args.steps / wall / 1e9
    result = {
        "metric": "KV swap round trip over the host link, GB/s (both directions)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.kv,
        "data": "synthetic",
        "config": {
            "workload": f"qwen3_8b_37x2304_swap{len(moved)}",
            "description": f"{args.kv} Hq=32 Hkv=8 d=128 B=16, {L} layers, {len(moved)} of 37 sequences x 2304 "
                           "tokens swapped out and back in per step",
            "frame_bytes": F,
            "frames_per_direction": blocks,
            "bytes_per_direction": nbytes,
            "staging_bytes": int(pool.staging.numel()),
        },
        "swap_out_ms": round(out_ms, 3),
        "swap_in_ms": round(in_ms, 3),
        "swap_out_gbs": round(gbs_out, 2),
        "swap_in_gbs": round(gbs_in, 2),
        "plain_pinned_copy_gbs": {"out": round(plain_out, 2), "in": round(plain_in, 2)},
        "fill_seconds": round(t_fill, 2),
        "roofline": {
            "bound": "host-link",
            "achieved": round(min(gbs_out, gbs_in), 2),
            "peak": PCIE_GEN5_X16_GBS,
            "unit": "GB/s",
            "frac": round(min(gbs_out, gbs_in) / PCIE_GEN5_X16_GBS, 4),
            "traffic": None,
            "kernel": "kv_seq_swap_out / kv_seq_swap_in (staging copy kernel + DMA), slower direction",
            "algorithmic_bytes_per_launch": nbytes,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = swap_cpu_baseline(args)
    print(json.dumps(result), flush=True)


def swap_cpu_baseline(args):
    """The oracle's swap of one sequence (bookkeeping plus its store's block copies), repeated."""
    from synth import workloads
    from oracle.runner import OracleReplay

    cores = 1
    wl = workloads.qwen_independent()
    ref = OracleReplay(wl, writers={0}).run()
    ref.bm.attach_host(200)
    n = ref.bm.length(0)
    nbytes = -(-n // wl.block_size) * wl.block_size * 2 * wl.num_kv_heads * wl.head_dim * wl.elem_bytes
    reps = 0
    t0 = time.perf_counter()
    while True:
        ref.store.to_host(ref.bm.swap_out(0))
        ref.store.from_host(ref.bm.swap_in(0))
        reps += 1
        if time.perf_counter() - t0 >= args.cpu_seconds:
            break
    wall = time.perf_counter() - t0
    return {
        "value": round(2 * nbytes * reps / wall / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"the oracle's swap out and back in of sequence 0 (2304 tokens, one layer), repeated {reps} "
                  f"times in {wall:.1f} s",
    }


def kernel_source_sha256(sources):
    import hashlib

    h = hashlib.sha256()
    for name in sources:
        with open(os.path.join(ROOT, "pagedattention_decode_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload, sources=DECODE_SOURCES, key="traffic_bytes_per_launch"):
    """HBM bytes per launch of the kernel streaming the cache (key
    traffic_bytes_per_launch) or per whole call (traffic_bytes_per_call) from
    the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary of this workload;
    None when there is none or the kernel sources changed since it was taken."""
    rec = traffic_record(workload, sources)
    return rec.get(key) if rec else None


def traffic_record(workload, sources=DECODE_SOURCES):
    """The committed counter summary of this workload (profiles/hbm_traffic_<workload>.json),
    or None when there is none or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if kernel_source_sha256(sources) != rec.get("kernel_source_sha256"):
        return None
    return rec


def traffic_ratio(workload, sources=DECODE_SOURCES, key="traffic_bytes_per_launch"):
    """HBM bytes over algorithmic bytes, both from the counter run itself (its contexts may be
    shorter than those of a longer bench run, so the ratio is the size-independent figure)."""
    rec = traffic_record(workload, sources)
    if not rec or not rec.get(key) or not rec.get("algorithmic_bytes_per_launch"):
        return None
    return rec[key] / rec["algorithmic_bytes_per_launch"]


# ---- summaries of rocprofv3 output for profiles/ ---------------------------

def short_kernel_name(name):
    """attn_mfma_kernel from 'void pagedkv::(anonymous namespace)::attn_mfma_kernel<...>(...)'."""
    head = name.replace("(anonymous namespace)::", "")
    head = head[5:] if head.startswith("void ") else head
    head = head.split("<", 1)[0].split("(", 1)[0]
    return head.rsplit("::", 1)[-1]


def read_csv_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def find_csv(run_dir, suffix):
    for dirpath, _, files in os.walk(run_dir):
        for fn in files:
            if fn.endswith(suffix):
                return os.path.join(dirpath, fn)
    raise FileNotFoundError(f"no *{suffix} under {run_dir}")


def bench_line(log_path):
    with open(log_path) as f:
        lines = [ln for ln in f.read().splitlines() if ln.startswith("{")]
    return json.loads(lines[-1]) if lines else None


def counter_kib_per_dispatch(run_dir, counter):
    """Mean counter value per dispatch, by short kernel name."""
    per = {}
    for r in read_csv_rows(find_csv(run_dir, "counter_collection.csv")):
        if r["Counter_Name"] != counter:
            continue
        per.setdefault(short_kernel_name(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in per.items()}


def summary_command():
    """This summary's own command line, with the output directory shown as <dir>."""
    import shlex
    args = sys.argv[1:]
    for i, x in enumerate(args[:-1]):
        if x in ("--summarize-counters", "--summarize-trace", "--summarize-activity"):
            args[i + 1] = "<out>" if x == "--summarize-trace" else "<dir>"
    return "python3 bench.py " + " ".join(shlex.quote(x) for x in args)


def summarize_counters(a):
    """--summarize-counters: FETCH_SIZE / WRITE_SIZE runs of a workload and of
    the plain-copy calibration -> profiles/hbm_traffic_<workload>.json and a
    markdown table.  Reads a directory holding pmc_<name>_{FETCH,WRITE}_SIZE/
    and pmc_cal_{FETCH,WRITE}_SIZE/ (with their .log files)."""
    d, name, wl = a.summarize_counters, a.summary_name, a.summary_workload
    kernels = a.summary_kernels.split(",")
    sources = tuple(a.summary_sources.split(","))
    fetch = counter_kib_per_dispatch(os.path.join(d, f"pmc_{name}_FETCH_SIZE"), "FETCH_SIZE")
    write = counter_kib_per_dispatch(os.path.join(d, f"pmc_{name}_WRITE_SIZE"), "WRITE_SIZE")
    cal_f = counter_kib_per_dispatch(os.path.join(d, "pmc_cal_FETCH_SIZE"), "FETCH_SIZE")
    cal_w = counter_kib_per_dispatch(os.path.join(d, "pmc_cal_WRITE_SIZE"), "WRITE_SIZE")
    cal = bench_line(os.path.join(d, "pmc_cal_FETCH_SIZE.log"))["copy_calibration_bytes_per_copy"]
    copy_f = max(cal_f.values())[0]
    copy_w = max(cal_w.values())[0]
    f_scale = cal / (copy_f * 1024)  # the copy reads cal bytes
    w_scale = cal / (copy_w * 1024)  # and writes cal bytes
    line = bench_line(os.path.join(d, f"pmc_{name}_FETCH_SIZE.log"))
    alg = line["roofline"].get("algorithmic_bytes_per_launch")
    flops = line["roofline"].get("algorithmic_flops_per_launch")
    per_kernel = {k: (fetch[k][0] * 1024 * f_scale, write.get(k, (0.0, 0))[0] * 1024 * w_scale) for k in kernels}
    main_k = kernels[0]
    rec = {
        "workload": wl,
        "kernel_source_sha256": kernel_source_sha256(sources),
        "sources": list(sources),
        "kernel": main_k,
        "traffic_bytes_per_launch": int(round(sum(per_kernel[main_k]))),
        "traffic_bytes_per_call": int(round(sum(sum(v) for v in per_kernel.values()))),
        "fetch_scale": f_scale,
        "write_scale": w_scale,
        "fetch_kib": {k: fetch[k][0] for k in kernels},
        "write_kib": {k: write.get(k, (0.0, 0))[0] for k in kernels},
        "algorithmic_bytes_per_launch": alg,
    }
    out_json = os.path.join(ROOT, "profiles", f"hbm_traffic_{wl}.json")
    with open(out_json, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    bench_args = a.summary_command
    md = [f"# HBM traffic counters: {a.summary_title}", "",
          "Commands (from the repository root, one pass per counter, each in a run of its own):", "", "```"]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        md.append(f"timeout -s KILL 150 rocprofv3 --pmc {c} --output-format csv -d <out> -o run -- "
                  f"python3 bench.py {bench_args}")
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        md.append(f"timeout -s KILL 150 rocprofv3 --pmc {c} --output-format csv -d <out> -o run -- "
                  f"python3 bench.py --copy-calibration {cal >> 20}")
    md += ["```", "", "Summarised from the four output directories (as `<dir>/pmc_<name>_<counter>/`, with each "
           f"run's stdout in `<dir>/pmc_<name>_<counter>.log`) by `{summary_command()}`.", "",
           f"Kernel sources sha256 ({', '.join(sources)}): `{rec['kernel_source_sha256']}`", "",
           f"Calibration with a plain device copy of {cal >> 20} MiB (`__amd_rocclr_copyBuffer`, as many bytes "
           f"read as written): FETCH_SIZE reads {copy_f:.1f} KiB per copy, WRITE_SIZE {copy_w:.1f} KiB, so bytes = "
           f"KiB x 1024 x {f_scale:.4f} (fetch) and x {w_scale:.4f} (write).", "",
           "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | fetched bytes (calibrated) | "
           "written bytes (calibrated) |", "|---|---|---|---|---|---|"]
    for k in kernels:
        md.append(f"| `{k}` | {fetch[k][1]} | {fetch[k][0]:.1f} | {write.get(k, (0.0, 0))[0]:.1f} | "
                  f"{per_kernel[k][0]:,.0f} | {per_kernel[k][1]:,.0f} |")
    if alg:
        md += ["", f"Algorithmic bytes per launch in the FETCH_SIZE run (K/V as stored, q, out, table entries): "
               f"{alg:,} B.  `{main_k}` moves {rec['traffic_bytes_per_launch']:,} B per launch "
               f"({rec['traffic_bytes_per_launch'] / alg:.4f} x algorithmic); the whole call "
               f"({', '.join(kernels)}) {rec['traffic_bytes_per_call']:,} B "
               f"({rec['traffic_bytes_per_call'] / alg:.4f} x)."]
    else:  # a matrix-bound launch: its roofline counts flops
        md += ["", f"`{main_k}` moves {rec['traffic_bytes_per_launch']:,} B per launch for {flops:,} flops "
               f"({flops / rec['traffic_bytes_per_launch']:.0f} flop/B); the whole call "
               f"({', '.join(kernels)}) {rec['traffic_bytes_per_call']:,} B."]
    out_md = os.path.join(ROOT, "profiles", f"{a.summary_file}.md")
    with open(out_md, "w") as f:
        f.write("\n".join(md) + "\n")
    print(out_json)
    print(out_md)


ACTIVITY_PASSES = ("SQ_INSTS_VALU SQ_INSTS_MFMA SQ_WAVE_CYCLES SQ_BUSY_CYCLES",
                   "SQ_ACTIVE_INST_VALU SQ_VALU_MFMA_BUSY_CYCLES SQ_WAIT_INST_ANY SQ_ACTIVE_INST_VMEM")


def summarize_activity(a):
    """--summarize-activity: per storage kind, two rocprofv3 --pmc passes of the
    same bench command (ACTIVITY_PASSES) -> a markdown table in profiles/:
    vector-ALU and matrix instructions per 16-token tile of the split-K kernel,
    and the shares of the waves' cycles spent issuing vector-ALU instructions
    and waiting."""
    d = a.summarize_activity
    rows_md = []
    for kind in a.summary_kinds.split(","):
        per = {}
        n_disp = None
        for i in (1, 2):
            vals = {}
            for r in read_csv_rows(find_csv(os.path.join(d, f"act_{kind}_{i}"), "counter_collection.csv")):
                if short_kernel_name(r["Kernel_Name"]) != "attn_mfma_kernel":
                    continue
                vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            for c, v in vals.items():
                per[c] = sum(v) / len(v)
                n_disp = len(v)
        line = bench_line(os.path.join(d, f"act_{kind}_1.log"))
        cfg = line["config"]
        tiles = cfg["sequences"] * cfg["context_tokens_first_step"] / 16 * 8  # 8 kv heads
        kv = kind.split("-")[0]
        wps = 1 if kv == "bf16" else 2
        valu_share = per["SQ_ACTIVE_INST_VALU"] / per["SQ_WAVE_CYCLES"]
        rows_md.append(f"| {kind} | {n_disp} | {per['SQ_INSTS_VALU'] / tiles:.1f} | {per['SQ_INSTS_MFMA'] / tiles:.1f} | "
                       f"{valu_share:.3f} | {wps} | {valu_share * wps:.2f} | "
                       f"{per['SQ_WAIT_INST_ANY'] / per['SQ_WAVE_CYCLES']:.3f} | {line['attn_kernel_us']} |")
    bench_args = a.summary_command
    md = [f"# Vector-ALU and matrix-core activity: {a.summary_title}", "",
          "Commands (from the repository root; two passes per storage kind <kind>, each a run of its own):", "",
          "```"]
    for kind in a.summary_kinds.split(","):
        kv, _, kern = kind.partition("-")  # <storage>[-<kernel>]
        kern_arg = f" --kernel {kern}" if kern else ""
        for i, pas in enumerate(ACTIVITY_PASSES, 1):
            md.append(f"timeout -s KILL 200 rocprofv3 --pmc {pas} --output-format csv -d <dir>/act_{kind}_{i} -o run "
                      f"-- python3 bench.py {bench_args} --kv {kv}{kern_arg} --steps 2 --warmup 1")
    md += ["```", "", f"Summarised by `{summary_command()}` (each run's stdout in `<dir>/act_<kind>_<pass>.log`).", "",
           "Per 16-token tile of one kv head (a wave's unit of work) in `attn_mfma_kernel`. `SQ_ACTIVE_INST_VALU` "
           "over `SQ_WAVE_CYCLES` is the share of a wave's cycles spent issuing vector-ALU instructions; times the "
           "waves per SIMD it estimates how busy each SIMD's vector ALU is. `SQ_WAIT_INST_ANY` over `SQ_WAVE_CYCLES` "
           "is the share spent waiting (mostly on memory).", "",
           "| storage[-kernel] | dispatches | VALU instructions per tile | MFMA per tile | VALU share of wave cycles | "
           "waves per SIMD | SIMD VALU busy (est.) | waiting share | kernel us (this run) |",
           "|---|---|---|---|---|---|---|---|---|"] + rows_md
    out_md = os.path.join(ROOT, "profiles", f"{a.summary_file}.md")
    with open(out_md, "w") as f:
        f.write("\n".join(md) + "\n")
    print(out_md)


def summarize_trace(a):
    """--summarize-trace: a rocprofv3 --kernel-trace --stats run (and the bench
    line it printed, <dir>.json) -> a markdown table in profiles/."""
    d = a.summarize_trace
    rows = read_csv_rows(find_csv(d, "kernel_stats.csv"))
    sources = tuple(a.summary_sources.split(","))
    md = [f"# Kernel trace: {a.summary_title}", "", "Command (from the repository root, on one MI355X):", "", "```",
          f"rocprofv3 --kernel-trace --stats --output-format csv -d <out> -o run -- python3 bench.py "
          f"{a.summary_command}", "```", "",
          f"Summarised from `<out>` (the run's stdout in `<out>.json`) by `{summary_command()}`.", "",
          f"Kernel sources sha256 ({', '.join(sources)}): `{kernel_source_sha256(sources)}`", "",
          "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for r in rows:
        md.append(f"| `{r['Name'][:100]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                  f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    line = bench_line(d.rstrip("/") + ".json")
    if line:
        r = line["roofline"]
        md += ["", "Bench line of the same run (under the tracer, which slows launches): "
               f"value {line['value']} {line['unit']}; "
               f"kernel {line.get('attn_kernel_us')} us and call {line.get('attn_call_us')} us by the library's "
               f"timing events; roofline {r['kernel']}: {r['achieved']} {r['unit']} of {r['peak']} "
               f"({r['frac']})."]
    out_md = os.path.join(ROOT, "profiles", f"{a.summary_file}.md")
    with open(out_md, "w") as f:
        f.write("\n".join(md) + "\n")
    print(out_md)


# threads of the CPU baseline: the host cores available to this process, at most this many
# (one GPU's share of its box)
CPU_BASELINE_MAX_WORKERS = 16


def _decode_workload(name, kv):
    """The oracle's workload for the CPU baseline and its rows (batch indices)."""
    from dataclasses import replace

    from synth import workloads

    if name == "agentic_fork_64x33281":
        wl = workloads.agentic_fork(steps=1, layers=1)
        rows = list(range(16))  # the 16 branches of root 0 (32770 tokens each at step 0)
    else:
        wl = workloads.get_workload(name)
        rows = None
    if kv != "bf16":
        wl = replace(wl, kv_format=kv)
    return wl, rows


def _cpu_baseline_worker(task):
    """One single-threaded oracle: the fp64 decode attention of `rows` of the
    workload's first decode (layer 0), repeated for `seconds`.  Runs in a fresh
    interpreter (spawn), which never touches the GPU."""
    name, kv, rows, writers, seconds = task
    import time as _t

    from threadpoolctl import threadpool_limits

    from oracle.runner import OracleReplay

    wl, _ = _decode_workload(name, kv)
    with threadpool_limits(limits=1):
        ref = OracleReplay(wl, layers=[0], writers=set(writers)).run()
        lens = ref.decodes[0]["lengths"]
        tokens = sum(lens[r] for r in rows)
        reps = 0
        c0 = _t.process_time()
        t0 = _t.perf_counter()
        while True:
            ref.attention(0, 0, rows=rows)
            reps += 1
            if _t.perf_counter() - t0 >= seconds:
                break
        wall = _t.perf_counter() - t0
        cpu = _t.process_time() - c0
    return {"tokens": tokens, "rows": len(rows), "reps": reps, "wall": wall, "cpu": cpu}


def cpu_baseline(args):
    """The fp64 oracle (unchanged) timed on the host: the workload's sequences are
    dealt to single-threaded oracle processes, one per available core (at most
    one per sequence), which decode their sequences in parallel for
    --cpu-seconds; the rate is the sum of the processes' rates."""
    import multiprocessing as mp

    name = args.workload
    wl, rows = _decode_workload(name, args.kv)
    n_seqs = len(next(op for op in wl.ops if op[0] == "decode")[1])
    rows = list(range(n_seqs)) if rows is None else rows
    workers = max(1, min(len(os.sched_getaffinity(0)), CPU_BASELINE_MAX_WORKERS, len(rows)))
    shares = [rows[w::workers] for w in range(workers)]
    roots = {0} if name == "agentic_fork_64x33281" else set()  # branches read their root's blocks
    tasks = [(name, args.kv, share, sorted(set(share) | roots), args.cpu_seconds) for share in shares]
    with mp.get_context("spawn").Pool(workers) as pool:
        res = pool.map(_cpu_baseline_worker, tasks)
    kv_per_tok = 2 * wl.num_kv_heads * (wl.head_dim * wl.elem_bytes if args.kv == "bf16" else
                                        wl.head_dim * (8 if args.kv == "q8_0" else 4) // 8 + wl.head_dim // 16)
    gbs = sum(r["tokens"] * kv_per_tok * r["reps"] / r["wall"] for r in res) / 1e9
    tok_s = sum(r["rows"] * r["reps"] / r["wall"] for r in res)
    wall = max(r["wall"] for r in res)
    util = sum(r["cpu"] for r in res) / wall
    return {
        "value": round(gbs, 4),
        "unit": "GB/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"{wl.name}{'' if args.kv == 'bf16' else ' (' + args.kv + ' pool)'}: the oracle's decode "
                  f"attention (layer 0, first decode step) of {len(rows)} sequences dealt to {workers} "
                  f"single-threaded processes, each repeating its share for {wall:.1f} s "
                  f"({sum(r['reps'] for r in res)} repetitions in all)",
        "tokens_per_s_per_layer": round(tok_s, 3),
        "cpu_utilisation": round(util, 2),
        "cores_available": len(os.sched_getaffinity(0)),
    }


if __name__ == "__main__":
    main()
