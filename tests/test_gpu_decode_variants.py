"""GPU parity of two variants of the split-K decode kept for measurement.

* KV_KERNEL_MFMA_STAGED_TABLE stages each wave's block-table entries in LDS
  instead of reading them with one scalar load per tile.  It computes exactly
  what the matrix-core kernel computes, so its outputs are compared bit for bit
  with KV_KERNEL_MFMA, and with the float64 oracle at the bf16 bars.
* KV_KERNEL_VALU does the arithmetic with v_dot2_f32_bf16 instead of matrix
  instructions (different rounding order), so it is compared with the oracle
  at the bf16 bars.

Both keep the edge cases of the matrix-core kernel (a zero-length context
gives a zero row, an out-of-range entry a NaN row) and refuse the pools they
do not read.  Every test prints the case it runs before touching the GPU.
"""

import numpy as np
import pytest
import torch

from oracle.runner import OracleReplay
from pagedattention_decode_amd import binding as B
from synth import draws, workloads
from tests.gpu_harness import GpuRun
from tests.test_gpu_parity import (RAGGED, announce, check_outputs, compare_all_decodes, ragged_workload,
                                   small_fork_workload)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("partition", [0, 16, 48, 512, 4096])
def test_staged_table_matches_scalar_reads_and_oracle(partition):
    announce(f"LDS-staged table entries, ragged lengths {RAGGED}, partition {partition}")
    wl = ragged_workload(32, 8, 128, RAGGED)
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref, fill=-1,
                 opts=B.attention_options(partition_tokens=partition, kernel=B.KV_KERNEL_MFMA_STAGED_TABLE)).run()
    compare_all_decodes(run, ref)
    rec = run.decodes[0]
    tables = torch.from_numpy(rec["tables"]).cuda()
    lens = torch.from_numpy(rec["lengths"]).cuda()
    n = len(RAGGED)
    staged = run.decode(0, 0, tables, lens, n, opts=B.attention_options(
        partition_tokens=partition, kernel=B.KV_KERNEL_MFMA_STAGED_TABLE))
    scalar = run.decode(0, 0, tables, lens, n, opts=B.attention_options(
        partition_tokens=partition, kernel=B.KV_KERNEL_MFMA))
    assert torch.equal(staged, scalar), "the staged-table variant differs from the scalar-read kernel"


def test_staged_table_37x2304_full():
    announce("LDS-staged table entries, Qwen3-8B-shaped layer, 37 x 2304 tokens")
    wl = workloads.qwen_independent()
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref, opts=B.attention_options(kernel=B.KV_KERNEL_MFMA_STAGED_TABLE)).run()
    compare_all_decodes(run, ref)


def test_staged_table_edge_cases_and_refusals():
    announce("LDS-staged table entries: zero-length context, out-of-range entry, unsupported pools")
    wl = ragged_workload(32, 8, 128, [40, 40, 40])
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref, fill=-1).run()
    tables = torch.from_numpy(run.decodes[0]["tables"]).cuda()
    lens = torch.from_numpy(run.decodes[0]["lengths"]).cuda()
    lens[1] = 0
    tables[2, 1] = wl.num_blocks + 5
    for part in (16, 0):
        out = run.decode(0, 0, tables, lens, 3, opts=B.attention_options(
            partition_tokens=part, kernel=B.KV_KERNEL_MFMA_STAGED_TABLE))
        o = out.double().cpu().numpy()
        check_outputs(o[:1], ref.attention(0, 0, rows=[0]), wl.dtype, "row 0 unaffected")
        assert (o[1] == 0).all()
        assert np.isnan(o[2]).all()
    # pools the variant does not read are refused, not silently run another way
    f32 = small_fork_workload(draws.F32, 4, 64)
    r2 = GpuRun(f32)
    with pytest.raises(B.KVError) as e:
        r2.pool.decode(0, torch.zeros((1, 4, 64), dtype=torch.int32, device="cuda"),
                       torch.zeros((1, 4, 64), dtype=torch.int32, device="cuda"),
                       torch.zeros((1, 2), dtype=torch.int32, device="cuda"),
                       torch.ones((1,), dtype=torch.int32, device="cuda"), 4,
                       opts=B.attention_options(kernel=B.KV_KERNEL_MFMA_STAGED_TABLE))
    assert e.value.status == B.KV_ERR_UNSUPPORTED


# ---------------------------------------------------------------------------
# the vector-ALU split-K variant (KV_KERNEL_VALU): same runs, ring and merge as
# the matrix-core kernel, v_dot2 arithmetic; checked against the oracle
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("hq", [32, 64])
@pytest.mark.parametrize("partition", [0, 48, 512, 4096])
def test_valu_variant_matches_oracle(hq, partition):
    announce(f"vector-ALU split-K kernel, Hq={hq} Hkv=8 d=128, ragged lengths {RAGGED}, partition {partition}")
    wl = ragged_workload(hq, 8, 128, RAGGED)
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref, fill=-1,
                 opts=B.attention_options(partition_tokens=partition, kernel=B.KV_KERNEL_VALU)).run()
    compare_all_decodes(run, ref)


def test_valu_variant_37x2304_full_and_edges():
    announce("vector-ALU split-K kernel: 37 x 2304 layer; zero-length context, out-of-range entry, refusals")
    wl = workloads.qwen_independent()
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref, opts=B.attention_options(kernel=B.KV_KERNEL_VALU)).run()
    compare_all_decodes(run, ref)
    wl = ragged_workload(32, 8, 128, [40, 40, 40])
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref, fill=-1).run()
    tables = torch.from_numpy(run.decodes[0]["tables"]).cuda()
    lens = torch.from_numpy(run.decodes[0]["lengths"]).cuda()
    lens[1] = 0
    tables[2, 1] = wl.num_blocks + 5
    for part in (16, 0):
        o = run.decode(0, 0, tables, lens, 3, opts=B.attention_options(
            partition_tokens=part, kernel=B.KV_KERNEL_VALU)).double().cpu().numpy()
        check_outputs(o[:1], ref.attention(0, 0, rows=[0]), wl.dtype, "row 0 unaffected")
        assert (o[1] == 0).all()
        assert np.isnan(o[2]).all()
    # G = 2 is not one of the instantiated group sizes: refused
    wl2 = ragged_workload(16, 8, 128, [20])
    r2 = GpuRun(wl2).run()
    t = torch.from_numpy(r2.decodes[0]["tables"]).cuda()
    l_ = torch.from_numpy(r2.decodes[0]["lengths"]).cuda()
    q = torch.zeros((1, 16, 128), dtype=torch.int16, device="cuda")
    with pytest.raises(B.KVError) as e:
        r2.pool.decode(0, q, q.clone(), t, l_, 16, opts=B.attention_options(kernel=B.KV_KERNEL_VALU))
    assert e.value.status == B.KV_ERR_UNSUPPORTED
