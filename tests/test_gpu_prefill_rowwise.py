"""GPU parity of the row-wise multi-query path against the float64 oracle.

paged_attention_prefill sends the pools its multi-query kernels do not read --
f32, quantised q8_0 / q4_0 pools with d = 256 -- and calls that ask for the
generic kernel (here also on bf16 pools of block size 4 and 8) through one
decode query per chunk row: row j of a chunk of
c rows over a context of n tokens reads the first n - c + j + 1 keys.  Bars:
f32 within 1e-5 max abs; bf16 (and bf16 queries over quantised pools, against
the oracle's attention over code x scale) within 2e-2 max abs and 5e-3 per-row
relative L2.  Rows of contract violations are NaN.
"""

import numpy as np
import pytest
import torch

from oracle.runner import OracleReplay
from pagedattention_decode_amd import binding as B
from synth import draws, workloads
from tests.gpu_harness import GpuRun, attention_errors

pytestmark = pytest.mark.gpu

BF16_ABS, BF16_REL, F32_ABS = 2e-2, 5e-3, 1e-5


def announce(msg):
    print(f"\n[case] {msg}", flush=True)


def check(got, expect, dtype, what):
    max_abs, rel = attention_errors(got, expect)
    print(f"  {what}: max abs {max_abs:.3e}, max row rel-L2 {rel:.3e}", flush=True)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    if dtype == draws.F32:
        assert max_abs <= F32_ABS, what
    else:
        assert max_abs <= BF16_ABS and rel <= BF16_REL, what


def chunk_wl(prompts, chunk, history, hq=32, hkv=8, d=128, bs=16, dtype=draws.BF16, kv_format="", seed=71):
    """Histories appended in bulk, then the prompts prefilled chunk by chunk."""
    seqs = tuple(range(len(prompts)))
    ops = [("add", s) for s in seqs]
    if any(history):
        grow = tuple(s for s in seqs if history[s])
        ops.append(("append", grow, tuple(history[s] for s in grow)))
    done = [0] * len(prompts)
    while any(x < p for x, p in zip(done, prompts)):
        ids = tuple(s for s in seqs if done[s] < prompts[s])
        counts = tuple(min(chunk, prompts[s] - done[s]) for s in ids)
        ops.append(("prefill", ids, counts))
        for s, c in zip(ids, counts):
            done[s] += c
    blocks = sum(-(-(p + h) // bs) for p, h in zip(prompts, history)) + 7
    return workloads.Workload("rowwise", seed, dtype, 1, hq, hkv, d, bs, blocks, ops, kv_format=kv_format)


def compare_all(run, ref, dtype, what):
    for i in range(len(ref.prefills)):
        expect = ref.prefill_attention(i, 0)
        got = run.prefill_outputs[i][0].double().cpu().numpy()
        first = np.concatenate([[0], np.cumsum(ref.prefills[i]["counts"])])
        for b in expect:
            check(got[first[b]:first[b + 1]], expect[b], dtype, f"{what}: prefill {i} batch {b}")


def test_f32_pool():
    announce("f32 pool, Hq=4 Hkv=1 d=64 B=4: ragged chunks of 8 over ragged histories")
    wl = chunk_wl((13, 7, 30), 8, (5, 0, 9), hq=4, hkv=1, d=64, bs=4, dtype=draws.F32)
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref, fill=-1).run()
    compare_all(run, ref, draws.F32, "f32")


@pytest.mark.parametrize("bs", [4, 8])
def test_bf16_other_block_sizes(bs):
    announce(f"bf16 pool with B = {bs}, Hq=8 Hkv=2 d=64, the generic kernel asked for: chunks of 24")
    wl = chunk_wl((50, 24, 3), 24, (40, 17, 0), hq=8, hkv=2, d=64, bs=bs)
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref, fill=-1, opts=B.attention_options(kernel=B.KV_KERNEL_GENERIC)).run()
    compare_all(run, ref, draws.BF16, f"bf16 B={bs}")


def test_generic_kernel_asked_for():
    announce("bf16 B = 16 pool with the generic kernel asked for: chunks of 32")
    wl = chunk_wl((70, 33), 32, (100, 5))
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref, fill=-1, opts=B.attention_options(kernel=B.KV_KERNEL_GENERIC)).run()
    compare_all(run, ref, draws.BF16, "generic")


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
def test_quantised_pools(fmt):
    announce(f"{fmt} pool, d = 256: chunks of 16 over histories, through the matrix-core decode kernel")
    wl = chunk_wl((40, 33, 1), 16, (100, 17, 64), hq=16, hkv=4, d=256, kv_format=fmt)
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref).run()
    compare_all(run, ref, draws.BF16, fmt)


def test_quantised_rows_in_batches():
    announce("q8_0 pool, d = 256, one chunk of 4200 rows (two launches of the decode kernel), sampled rows")
    wl = chunk_wl((2100, 2100), 2100, (64, 30), hq=16, hkv=4, d=256, kv_format="q8_0")
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref).run()
    got = run.prefill_outputs[0][0].double().cpu().numpy()
    picks = [(0, 0), (0, 1), (0, 1000), (0, 2099), (1, 0), (1, 1994), (1, 1995), (1, 1996), (1, 2099)]
    first = [0, 2100]
    rows = [first[b] + j for b, j in picks]  # rows 4094, 4095, 4096 straddle the two launches
    check(got[rows], ref.prefill_rows(0, 0, picks), draws.BF16, "q8_0 sampled")


def test_contract_violations():
    announce("row-wise path (generic kernel asked for, B = 8): c > n, c > max_q_len and a bad table entry give "
             "NaN rows, nothing else")
    wl = chunk_wl((40, 40, 40), 40, (10, 10, 10), hq=8, hkv=2, d=64, bs=8)
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref, fill=-1, opts=B.attention_options(kernel=B.KV_KERNEL_GENERIC)).run()
    rec = run.prefills[0]
    tables = torch.from_numpy(rec["tables"]).cuda()
    lens = torch.from_numpy(rec["lengths"]).cuda()
    indptr = torch.tensor([0, 40, 80, 120], dtype=torch.int32, device="cuda")
    lens[1] = 30                      # 40 queries over 30 tokens: NaN rows
    tables[2, 3] = wl.num_blocks + 3  # positions 24..31: rows that see them are NaN
    out = run.prefill(0, 0, indptr, tables, lens, 40).double().cpu().numpy()
    expect = ref.prefill_attention(0, 0)
    check(out[0:40], expect[0], draws.BF16, "sequence 0")
    assert np.isnan(out[40:80]).all()
    # sequence 2: history 10, row j sees positions 0 .. 10 + j; block 3 holds 24..31
    check(out[80:94], expect[2][:14], draws.BF16, "sequence 2 rows before the bad block")
    assert np.isnan(out[94:120]).all()
    lens = torch.from_numpy(rec["lengths"]).cuda()
    tables = torch.from_numpy(rec["tables"]).cuda()
    out = run.prefill(0, 0, torch.tensor([0, 40, 80, 81], dtype=torch.int32, device="cuda"), tables, lens, 1)
    assert np.isnan(out.double().cpu().numpy()[0:80]).all()
    # the matrix-core kernel does not read f32 pools
    f32 = chunk_wl((4,), 4, (0,), hq=4, hkv=1, d=64, bs=4, dtype=draws.F32)
    r2 = GpuRun(f32).run()
    z = torch.zeros((4, 4, 64), dtype=torch.int32, device="cuda")
    with pytest.raises(B.KVError) as e:
        r2.pool.prefill(0, z, z.clone(), torch.tensor([0, 4], dtype=torch.int32, device="cuda"),
                        torch.zeros((1, 2), dtype=torch.int32, device="cuda"),
                        torch.full((1,), 4, dtype=torch.int32, device="cuda"), 4, 4,
                        opts=B.attention_options(kernel=B.KV_KERNEL_MFMA))
    assert e.value.status == B.KV_ERR_UNSUPPORTED
    torch.cuda.synchronize()
