"""GPU parity of the matrix-core decode over bf16 pools whose block size is not
16 (B = 4, 8, 32, 64), against the float64 oracle at the bf16 bar.

For B > 16 the kernel reads each table entry as B/16 tiles of 16 tokens; for
B < 16 a tile gathers 16/B entries, and only the entries holding tokens of the
context are read -- the last tile of a context may reach past the table's row,
which the ragged lengths below provoke on every sequence whose length is not a
multiple of 16.  The block-size trade-off ([KVM] block-size trade-off; [BT] §09)
makes B a deployment choice, so the fast kernel has to take every common one.
"""

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
