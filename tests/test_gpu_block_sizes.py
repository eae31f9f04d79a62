"""GPU parity of the matrix-core decode and of the multi-query kernels (chunked
prefill) over bf16 pools whose block size is not 16 (B = 4, 8, 32, 64), against
the float64 oracle at the bf16 bar.

For B > 16 the kernel reads each table entry as B/16 tiles of 16 tokens; for
B < 16 a tile gathers 16/B entries, and only the entries holding tokens of the
context are read -- the last tile of a context may reach past the table's row,
which the ragged lengths below provoke on every sequence whose length is not a
multiple of 16.  The block-size trade-off ([KVM] block-size trade-off; [BT] §09)
makes B a deployment choice, so the fast kernel has to take every common one.
"""

import dataclasses
import math

import numpy as np
import pytest
import torch

from oracle.attention import decode_attention
from oracle.runner import OracleReplay
from pagedattention_decode_amd import binding as B
from synth import draws, workloads
from tests.gpu_harness import GpuRun, attention_errors

pytestmark = pytest.mark.gpu

BF16_ABS, BF16_REL = 2e-2, 5e-3
BLOCK_SIZES = (4, 8, 32, 64)
MFMA = B.KV_KERNEL_MFMA


def announce(msg):
    print(f"\n[case] {msg}", flush=True)


def check(got, expect, what):
    max_abs, rel = attention_errors(got, expect)
    print(f"  {what}: max abs {max_abs:.3e}, max row rel-L2 {rel:.3e}", flush=True)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert max_abs <= BF16_ABS and rel <= BF16_REL, what


def ragged(bs, lengths, hq=32, hkv=8, d=128, seed=43):
    seqs = tuple(range(len(lengths)))
    ops = [("add", s) for s in seqs] + [("append", seqs, tuple(lengths)), ("decode", seqs)]
    blocks = sum(-(-n // bs) for n in lengths) + 7
    return workloads.Workload(f"ragged_b{bs}", seed, draws.BF16, 1, hq, hkv, d, bs, blocks, ops)


LENGTHS = [1, 2, 3, 4, 5, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 257, 511, 1000, 2049]


@pytest.mark.parametrize("bs", BLOCK_SIZES)
def test_ragged_lengths_and_partitions(bs):
    announce(f"B={bs}: ragged lengths {LENGTHS}, partitions auto / B / 4 lcm(B, 16) / 512, NaN background")
    wl = ragged(bs, LENGTHS)
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref, fill=-1, opts=B.attention_options(kernel=MFMA)).run()
    expect = ref.attention(0, 0)
    check(run.decode_outputs[0][0].double().cpu().numpy(), expect, f"B={bs} auto")
    rec = run.decodes[0]
    tables = torch.from_numpy(rec["tables"]).cuda()
    lens = torch.from_numpy(rec["lengths"]).cuda()
    for part in (bs, 4 * math.lcm(bs, 16), 512):
        out = run.decode(0, 0, tables, lens, len(LENGTHS), opts=B.attention_options(kernel=MFMA, partition_tokens=part))
        check(out.double().cpu().numpy(), expect, f"B={bs} partition {part}")


@pytest.mark.parametrize("bs", BLOCK_SIZES)
@pytest.mark.parametrize("hq,hkv,d", [(8, 8, 128), (64, 8, 128), (16, 1, 128), (32, 8, 64), (16, 4, 256)])
def test_head_shapes(bs, hq, hkv, d):
    announce(f"B={bs}: head shapes Hq={hq} Hkv={hkv} d={d}")
    wl = ragged(bs, [1, 7, 16, 33, 300, 700], hq=hq, hkv=hkv, d=d)
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref, fill=-1, opts=B.attention_options(kernel=MFMA, partition_tokens=128)).run()
    check(run.decode_outputs[0][0].double().cpu().numpy(), ref.attention(0, 0), f"B={bs} Hq={hq} Hkv={hkv} d={d}")


@pytest.mark.parametrize("bs", BLOCK_SIZES)
def test_bad_entries_and_empty_contexts(bs):
    announce(f"B={bs}: context 0 -> zero row; a table entry outside the pool -> NaN row, never read")
    wl = ragged(bs, [40, 40, 40, 40])
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref, fill=-1).run()
    tables = torch.from_numpy(run.decodes[0]["tables"]).cuda()
    lens = torch.from_numpy(run.decodes[0]["lengths"]).cuda()
    lens[1] = 0
    tables[2, (24 // bs)] = wl.num_blocks + 5  # the entry holding token 24
    # entries past a context (sequence 3 keeps 20 tokens) are never read, whatever they hold
    lens[3] = 20
    tables[3, -(-20 // bs):] = -7
    q = draws.bits_to_f64(run.query_bits(0, 0, 4), wl.dtype)
    k, v = ref.gather_f64(0, ref.decodes[0]["tables"][3], 20)
    expect3 = decode_attention(q[3], k, v)[None]
    for part in (0, 512):
        out = run.decode(0, 0, tables, lens, 4, opts=B.attention_options(kernel=MFMA, partition_tokens=part))
        o = out.double().cpu().numpy()
        check(o[:1], ref.attention(0, 0, rows=[0]), f"B={bs} row 0")
        assert (o[1] == 0).all()
        assert np.isnan(o[2]).all()
        check(o[3:4], expect3, f"B={bs} row 3 over its first 20 tokens")


def test_qwen3_8b_37x2304_at_block_size_32():
    announce("Qwen3-8B-shaped layer, 37 x 2304 tokens, bf16, B=32, default launch")
    base = workloads.qwen_independent()
    from dataclasses import replace
    wl = replace(base, name="qwen3_8b_37x2304_b32", block_size=32, num_blocks=37 * 72 + 40)
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref).run()
    check(run.decode_outputs[0][0].double().cpu().numpy(), ref.attention(0, 0), "37 x 2304, B=32")


# ---- multi-query attention (chunked prefill) over pools of block size 4 .. 64 ----
# The multi-query kernels read 16-token tiles: for B > 16 tile j is sub-tile
# j % (B/16) of table entry j / (B/16) (partitions of 48 tokens make pairs of
# tiles that straddle two entries); for B < 16 a tile gathers 16/B entries.

def chunks_b(bs, prompts, chunk, history, hq=32, hkv=8, d=128, seed=47):
    seqs = tuple(range(len(prompts)))
    ops = [("add", s) for s in seqs]
    grow = tuple(s for s in seqs if history[s])
    if grow:
        ops.append(("append", grow, tuple(history[s] for s in grow)))
    done = [0] * len(prompts)
    while any(x < p for x, p in zip(done, prompts)):
        ids = tuple(s for s in seqs if done[s] < prompts[s])
        counts = tuple(min(chunk, prompts[s] - done[s]) for s in ids)
        ops.append(("prefill", ids, counts))
        for s, c in zip(ids, counts):
            done[s] += c
    blocks = sum(-(-(p + h) // bs) for p, h in zip(prompts, history)) + 7
    return workloads.Workload(f"chunks_b{bs}", seed, draws.BF16, 1, hq, hkv, d, bs, blocks, ops)


def compare_prefills(run, ref, what):
    for i in range(len(ref.prefills)):
        expect = ref.prefill_attention(i, 0)
        got = run.prefill_outputs[i][0].double().cpu().numpy()
        first = np.concatenate([[0], np.cumsum(ref.prefills[i]["counts"])])
        for b in expect:
            check(got[first[b]:first[b + 1]], expect[b], f"{what} prefill {i} seq {ref.prefills[i]['seq_ids'][b]}")


@pytest.mark.parametrize("bs", (4, 8, 32, 64))
@pytest.mark.parametrize("partition", [0, 16, 48, 4096])
def test_multi_query_ragged_chunks(bs, partition):
    announce(f"multi-query, B={bs}: prompts (700, 33, 1, 517, 16, 130) in chunks of 100, partition {partition}")
    wl = chunks_b(bs, (700, 33, 1, 517, 16, 130), 100, (0, 40, 3, 17, 0, 1))
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref, fill=-1, opts=B.attention_options(partition_tokens=partition)).run()
    compare_prefills(run, ref, f"B={bs} P={partition}")


@pytest.mark.parametrize("bs", (4, 8, 32, 64))
@pytest.mark.parametrize("hq,hkv,d", [(8, 8, 128), (64, 8, 128), (16, 1, 128), (32, 8, 64), (16, 4, 256),
                                      (12, 4, 64)])
def test_multi_query_head_shapes(bs, hq, hkv, d):
    announce(f"multi-query, B={bs}, Hq={hq} Hkv={hkv} d={d}: prompts (97, 16, 5) in chunks of 40")
    wl = chunks_b(bs, (97, 16, 5), 40, (20, 0, 300), hq=hq, hkv=hkv, d=d)
    ref = OracleReplay(wl).run()
    for part in (0, 32):
        run = GpuRun(wl, ref=ref, fill=-1, opts=B.attention_options(partition_tokens=part)).run()
        compare_prefills(run, ref, f"B={bs} P={part}")


@pytest.mark.parametrize("bs", (4, 8, 32, 64))
def test_multi_query_last_chunk_of_8k_prompts_sampled(bs):
    announce(f"multi-query, B={bs}: 16 x (7680 cached + 512-token chunk), default launch, rows sampled")
    base = workloads.prefill_last_chunk()
    wl = dataclasses.replace(base, block_size=bs, num_blocks=-(-base.num_blocks * 16 // bs) + 16)
    sample = [0, 7, 15]
    ref = OracleReplay(wl, writers=sample).run()
    run = GpuRun(wl, ref=ref, writers=sample).run()
    got = run.prefill_outputs[0][0].double().cpu().numpy()
    picks = [(b, j) for b in sample for j in (0, 1, 15, 16, 63, 64, 255, 256, 510, 511)]
    rows = [b * 512 + j for b, j in picks]
    check(got[rows], ref.prefill_rows(0, 0, picks), f"B={bs} last chunk sampled")


@pytest.mark.parametrize("bs", (8, 32))
def test_multi_query_bad_entry(bs):
    announce(f"multi-query, B={bs}: a table entry outside [0, N) gives NaN rows for the rows that see it")
    wl = chunks_b(bs, (40, 40), 40, (10, 50))
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref, fill=-1).run()
    rec = run.prefills[0]
    tables = torch.from_numpy(rec["tables"]).cuda()
    lens = torch.from_numpy(rec["lengths"]).cuda()
    tables[1, 64 // bs] = wl.num_blocks + 3  # sequence 1: positions from 64 (history 50, rows j >= 14 see them)
    indptr = torch.tensor([0, 40, 80], dtype=torch.int32, device="cuda")
    out = run.prefill(0, 0, indptr, tables, lens, 40).double().cpu().numpy()
    expect = ref.prefill_attention(0, 0)
    check(out[0:40], expect[0], "sequence 0 unaffected")
    assert np.isnan(out[40 + 14:80]).all()
    for j in range(14):
        row = out[40 + j]
        if not np.isnan(row).all():
            check(row[None], expect[1][j][None], f"sequence 1 row {j}")
    torch.cuda.synchronize()
