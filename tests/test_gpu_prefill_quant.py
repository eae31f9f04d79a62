"""GPU parity of multi-query attention over quantised pools (q8_0 / q4_0, d = 64
and 128) -- chunked prefill and draft verification through the multi-query
kernel for quantised tiles -- against the float64 oracle's attention over
code x scale.

Bars as for bf16: max abs error 2e-2 and per-row relative L2 error 5e-3.
Outputs, workspace and the pool's unwritten bytes start as NaN bytes (the half
scales of unwritten slots are NaN), so an unwritten row, or a masked slot that
is not weighted 0, fails.  Every test prints its case before touching the GPU.
"""

import dataclasses

import numpy as np
import pytest
import torch

from oracle.runner import OracleReplay
from pagedattention_decode_amd import binding as B
from synth import draws, workloads
from tests.gpu_harness import GpuRun, attention_errors

pytestmark = pytest.mark.gpu

BF16_ABS, BF16_REL = 2e-2, 5e-3
FMTS = ["q8_0", "q4_0"]


def announce(msg):
    print(f"\n[case] {msg}", flush=True)


def check(got, expect, what):
    max_abs, rel = attention_errors(got, expect)
    print(f"  {what}: max abs {max_abs:.3e}, max row rel-L2 {rel:.3e}", flush=True)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert max_abs <= BF16_ABS and rel <= BF16_REL, what


def quant_chunks(prompts, chunk, fmt, hq=32, hkv=8, d=128, history=None, seed=43):
    """Prompts prefilled chunk by chunk over a quantised pool; ``history`` tokens
    per prompt are appended first in bulk (no queries)."""
    seqs = tuple(range(len(prompts)))
    ops = [("add", s) for s in seqs]
    if history and any(history):
        grow = tuple(s for s in seqs if history[s])
        ops.append(("append", grow, tuple(history[s] for s in grow)))
    done = [0] * len(prompts)
    while any(x < p for x, p in zip(done, prompts)):
        ids = tuple(s for s in seqs if done[s] < prompts[s])
        counts = tuple(min(chunk, prompts[s] - done[s]) for s in ids)
        ops.append(("prefill", ids, counts))
        for s, c in zip(ids, counts):
            done[s] += c
    total = [p + (history[i] if history else 0) for i, p in enumerate(prompts)]
    blocks = sum(-(-t // 16) for t in total)
    return workloads.Workload("quant_chunks", seed, draws.BF16, 1, hq, hkv, d, 16, blocks + 9, ops, kv_format=fmt)


def compare_all(run, ref, what=""):
    for i in range(len(ref.prefills)):
        expect = ref.prefill_attention(i, 0)
        got = run.prefill_outputs[i][0].double().cpu().numpy()
        first = np.concatenate([[0], np.cumsum(ref.prefills[i]["counts"])])
        for b in expect:
            check(got[first[b]:first[b + 1]], expect[b], f"{what} prefill {i} seq {ref.prefills[i]['seq_ids'][b]}")


RAGGED_PROMPTS = (700, 33, 1, 517, 16, 130)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("partition", [0, 16, 64, 4096])
def test_ragged_chunks_and_partitions(fmt, partition):
    announce(f"{fmt}: prompts {RAGGED_PROMPTS} in chunks of 100 over 0..40 history tokens, partition {partition}")
    wl = quant_chunks(RAGGED_PROMPTS, 100, fmt, history=[0, 40, 3, 17, 0, 1])
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref, fill=-1, opts=B.attention_options(partition_tokens=partition)).run()
    compare_all(run, ref, f"{fmt} P={partition}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("hq,hkv,d", [(8, 8, 128), (64, 8, 128), (16, 1, 128), (32, 8, 64), (12, 4, 64),
                                      (48, 3, 128)])
def test_head_shapes(fmt, hq, hkv, d):
    announce(f"{fmt}: head shapes Hq={hq} Hkv={hkv} d={d}: prompts (97, 16, 5) in chunks of 40")
    wl = quant_chunks((97, 16, 5), 40, fmt, hq=hq, hkv=hkv, d=d, history=[20, 0, 300])
    ref = OracleReplay(wl).run()
    for part in (0, 32):
        run = GpuRun(wl, ref=ref, fill=-1, opts=B.attention_options(partition_tokens=part)).run()
        compare_all(run, ref, f"{fmt} P={part}")


@pytest.mark.parametrize("fmt", FMTS)
def test_last_chunk_of_8k_prompts_sampled(fmt):
    announce(f"{fmt}: 16 x (7680 cached + 512-token chunk), default launch; rows sampled in sequences 0, 7, 15")
    wl = dataclasses.replace(workloads.prefill_last_chunk(), kv_format=fmt)
    sample = [0, 7, 15]
    ref = OracleReplay(wl, writers=sample).run()
    run = GpuRun(wl, ref=ref, writers=sample).run()
    got = run.prefill_outputs[0][0].double().cpu().numpy()
    picks = [(b, j) for b in sample for j in (0, 1, 15, 16, 63, 64, 255, 256, 510, 511)]
    rows = [b * 512 + j for b, j in picks]
    check(got[rows], ref.prefill_rows(0, 0, picks), f"{fmt} last chunk sampled")


@pytest.mark.parametrize("fmt", FMTS)
def test_verify_8_drafts_full(fmt):
    announce(f"{fmt}: 16 x (8184 cached + 8 draft positions), default launch; every row checked")
    wl = dataclasses.replace(workloads.verify_drafts(), kv_format=fmt)
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref).run()
    got = run.prefill_outputs[0][0].double().cpu().numpy()
    picks = [(b, j) for b in range(16) for j in range(8)]
    check(got, ref.prefill_rows(0, 0, picks), f"{fmt} verify 16 x 8")


@pytest.mark.parametrize("fmt", FMTS)
def test_contract_violations_give_nan_rows(fmt):
    announce(f"{fmt}: chunk longer than its context or than max_q_len -> NaN rows; bad table entry -> NaN")
    wl = quant_chunks((40, 40, 40), 40, fmt, history=[10, 10, 10])
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref, fill=-1).run()
    rec = run.prefills[0]
    tables = torch.from_numpy(rec["tables"]).cuda()
    lens = torch.from_numpy(rec["lengths"]).cuda()
    indptr = torch.tensor([0, 40, 80, 120], dtype=torch.int32, device="cuda")
    lens[1] = 30                      # 40 queries over 30 tokens: NaN rows
    tables[2, 1] = wl.num_blocks + 3  # never dereferenced: NaN rows
    out = run.prefill(0, 0, indptr, tables, lens, 40).double().cpu().numpy()
    expect = ref.prefill_attention(0, 0)
    check(out[0:40], expect[0], f"{fmt} sequence 0 unaffected")
    assert np.isnan(out[40:80]).all()
    # rows of sequence 2 that see block 1 (position 10 + j >= 16) are NaN; an earlier row is
    # NaN when its query tile reads block 1 for another row, else exact
    assert np.isnan(out[86:120]).all()
    for j in range(6):
        row = out[80 + j]
        if not np.isnan(row).all():
            check(row[None], expect[2][j][None], f"{fmt} sequence 2 row {j}")
    lens = torch.from_numpy(rec["lengths"]).cuda()
    tables = torch.from_numpy(rec["tables"]).cuda()
    out = run.prefill(0, 0, torch.tensor([0, 40, 80, 81], dtype=torch.int32, device="cuda"), tables, lens, 1)
    assert np.isnan(out.double().cpu().numpy()[0:80]).all()
    torch.cuda.synchronize()
