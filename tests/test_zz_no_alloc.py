"""The allocation-free decode entry point (paged_attention_decode_static), for
callers that cannot allocate device memory, against paged_attention_decode
with a caller workspace: identical output bits on two calls in a row (the
second with fewer, shorter sequences, so it reads scratch the first left
behind), both within the bf16 bar of the float64 oracle; calls whose
workspace would exceed the static scratch are refused; the workspace entry
point is unchanged afterwards.
"""

import numpy as np
import pytest
import torch

from oracle.runner import OracleReplay
from pagedattention_decode_amd import binding as B
from synth import workloads
from tests.gpu_harness import GpuRun, attention_errors, bits_to_float_tensor, to_device_bits

pytestmark = pytest.mark.gpu

BF16_ABS, BF16_REL = 2e-2, 5e-3


def announce(msg):
    print(f"\n[case] {msg}", flush=True)


def ragged(lengths, hq=32, hkv=8, d=128, seed=71):
    seqs = tuple(range(len(lengths)))
    ops = [("add", s) for s in seqs] + [("append", seqs, tuple(lengths)), ("decode", seqs)]
    blocks = sum(-(-n // 16) for n in lengths) + 8
    return workloads.Workload("no_alloc", seed, "bf16", 1, hq, hkv, d, 16, blocks, ops)


def both_entry_points(run, ref, opts):
    rec = run.decodes[0]
    n = len(rec["seq_ids"])
    tables = torch.from_numpy(rec["tables"]).cuda()
    lens = torch.from_numpy(rec["lengths"]).cuda()
    q = to_device_bits(run.query_bits(0, 0, n))
    hq = run.wl.num_q_heads
    ws = torch.empty(max(run.pool.workspace_bytes(n, hq, tables.shape[1], opts), 1), dtype=torch.uint8,
                     device="cuda")
    assert ws.numel() <= B.paged_attention_static_scratch_bytes()
    out_ws = torch.full_like(q, -1)
    out_static = torch.full_like(q, -1)
    run.pool.decode(0, q, out_ws, tables, lens, hq, opts, ws)
    run.pool.decode_static(0, q, out_static, tables, lens, hq, opts)
    torch.cuda.synchronize()
    assert torch.equal(out_static, out_ws), "the static-scratch decode differs from the workspace decode"
    got = bits_to_float_tensor(out_static, "bf16").double().cpu().numpy()
    max_abs, rel = attention_errors(got, ref.attention(0, 0))
    print(f"  {n} sequences: bit-identical; vs oracle max abs {max_abs:.3e}, rel-L2 {rel:.3e}", flush=True)
    assert max_abs <= BF16_ABS and rel <= BF16_REL


@pytest.mark.parametrize("opts", [B.attention_options(), B.attention_options(partition_tokens=512),
                                  B.attention_options(kernel=B.KV_KERNEL_GENERIC, partition_tokens=256)],
                         ids=["mfma-auto", "mfma-512", "generic-256"])
def test_static_scratch_decode_equals_workspace_decode(opts):
    announce("allocation-free decode vs workspace decode: 37 x 2304 tokens, then 5 ragged shorter sequences")
    for lengths in ([2304] * 37, [1, 17, 300, 1000, 2049]):
        wl = ragged(lengths)
        ref = OracleReplay(wl).run()
        run = GpuRun(wl, ref=ref, fill=-1).run()
        both_entry_points(run, ref, opts)


def test_static_scratch_refuses_oversized_calls_and_leaves_the_workspace_path_alone():
    announce("allocation-free decode: a call needing more than the static scratch is refused")
    wl = ragged([40, 40])
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref).run()
    # one partition per block over 40000 table entries: the generic kernel's partials
    # (32 heads x 40000 partitions x (128 + 2) floats) are far above the scratch
    opts = B.attention_options(kernel=B.KV_KERNEL_GENERIC, partition_tokens=16)
    tables = torch.full((2, 40000), -1, dtype=torch.int32, device="cuda")
    tables[:, :3] = torch.from_numpy(run.decodes[0]["tables"][:, :3]).cuda()
    lens = torch.from_numpy(run.decodes[0]["lengths"]).cuda()
    assert run.pool.workspace_bytes(2, 32, 40000, opts) > B.paged_attention_static_scratch_bytes()
    q = to_device_bits(run.query_bits(0, 0, 2))
    out = torch.full_like(q, -1)
    with pytest.raises(B.KVError) as e:
        run.pool.decode_static(0, q, out, tables, lens, 32, opts)
    assert e.value.status == B.KV_ERR_INVALID and "static scratch" in str(e.value)
    assert (out == -1).all(), "a refused call wrote its output"
    both_entry_points(run, ref, B.attention_options())
