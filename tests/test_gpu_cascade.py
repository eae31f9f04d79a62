"""GPU parity of the read-once decode over shared prefixes (cascade) against the
float64 oracle, bf16 bar (over q8_0 / q4_0 pools against the oracle's attention
over code x scale).  The groups come from the library's own plan of the
host tables unless a test gives them; outputs and workspace start as NaN bytes.
The fork workload (4 roots x 16 forks, 512 steps, 36 layers) is checked with
the read-once decode beside the plain one in test_gpu_parity.py
(test_agentic_fork_sampled), so that its long replay runs once.
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle.runner import OracleReplay
from pagedattention_decode_amd import binding as B
from synth import draws, workloads
from tests.gpu_harness import GpuRun, attention_errors

pytestmark = pytest.mark.gpu

BF16_ABS, BF16_REL = 2e-2, 5e-3


def announce(msg):
    print(f"\n[case] {msg}", flush=True)


def check(got, expect, what):
    max_abs, rel = attention_errors(got, expect)
    print(f"  {what}: max abs {max_abs:.3e}, max row rel-L2 {rel:.3e}", flush=True)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert max_abs <= BF16_ABS and rel <= BF16_REL, what


def fork_workload(groups, layers=1, seed=61, hq=32, hkv=8, d=128):
    """groups: [(root_len, [suffix lengths of its forks])]; each root forks len(list) times
    (the first entry keeps the root), then every member appends its suffix."""
    ops, seqs, suffixes, blocks = [], [], [], 0
    sid = 0
    for root_len, sfx in groups:
        root = sid
        ops += [("add", root), ("append", (root,), (root_len,))]
        members = [root] + list(range(root + 1, root + len(sfx)))
        ops += [("fork", root, m) for m in members[1:]]
        seqs += members
        suffixes += list(sfx)
        blocks += -(-root_len // 16) + sum(-(-s // 16) + 1 for s in sfx)
        sid += len(sfx)
    grow = [(s, c) for s, c in zip(seqs, suffixes) if c > 0]
    if grow:
        ops.append(("append", tuple(s for s, _ in grow), tuple(c for _, c in grow)))
    ops.append(("decode", tuple(seqs)))
    return workloads.Workload("forks", seed, draws.BF16, layers, hq, hkv, d, 16, blocks + 16, ops)


def test_shared_prefix_16x8448_full():
    announce("16 x 8448 tokens sharing 6144: cascade decode vs oracle")
    wl = workloads.shared_prefix()
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref).run()
    gs, sb = run.pool.shared_prefix_plan(run.decodes[0]["seq_ids"])
    assert list(gs) == [0, 16] and list(sb) == [384]
    out = run.decode_cascade(0, 0).double().cpu().numpy()
    check(out, ref.attention(0, 0), "16 x 8448 cascade")


@pytest.mark.parametrize("partition", [0, 64, 512])
def test_ragged_groups(partition):
    announce(f"ragged fork groups, empty suffixes and singletons, partition {partition}, NaN background")
    groups = [(32, [0, 0, 5]), (100, [1, 17, 300, 0]), (7, [20]), (512, [16, 16, 16, 16, 33, 1000]), (48, [0])]
    wl = fork_workload(groups)
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref, fill=-1).run()
    gs, sb = run.pool.shared_prefix_plan(run.decodes[0]["seq_ids"])
    print("  plan", list(gs), list(sb), flush=True)
    assert max(sb) > 0 and min(np.diff(gs)) >= 1
    out = run.decode_cascade(0, 0, opts=B.attention_options(partition_tokens=partition)).double().cpu().numpy()
    check(out, ref.attention(0, 0), f"ragged groups P={partition}")


def test_no_sharing_equals_plain_decode():
    announce("independent sequences: every group a singleton, equal to the plain decode")
    wl = fork_workload([(300, [0]), (17, [0]), (1000, [0])])
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref).run()
    out = run.decode_cascade(0, 0).double().cpu().numpy()
    check(out, ref.attention(0, 0), "singletons")


def test_contract_violations_give_nan_rows():
    announce("cascade: a member whose table differs, a prefix longer than a context, a group over max_group")
    wl = fork_workload([(64, [0, 3, 20]), (80, [2, 2])])
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref, fill=-1).run()
    rec = run.decodes[0]
    gs, sb = run.pool.shared_prefix_plan(rec["seq_ids"])
    assert list(gs) == [0, 3, 5] and list(sb) == [4, 5]
    expect = ref.attention(0, 0)
    # member 2's first table entry replaced: only its rows are NaN
    tables = rec["tables"].copy()
    tables[2, 0] = tables[2, 1]
    out = run.decode_cascade(0, 0, tables=tables).double().cpu().numpy()
    assert np.isnan(out[2]).all()
    check(out[[0, 1, 3, 4]], expect[[0, 1, 3, 4]], "other members")
    # a shared count beyond the group's contexts: the group's rows are NaN
    out = run.decode_cascade(0, 0, plan=(gs, np.array([4, 7], np.int32))).double().cpu().numpy()
    assert np.isnan(out[3:5]).all()
    check(out[:3], expect[:3], "group 0")
    # a prefix the first member's context does not cover: member 2 (84 tokens) would, but the
    # first (64) sets the prefix length, so the whole group is NaN
    out = run.decode_cascade(0, 0, plan=(gs, np.array([5, 5], np.int32))).double().cpu().numpy()
    assert np.isnan(out[:3]).all()
    check(out[3:5], expect[3:5], "group 1, 5 shared blocks")
    # max_group smaller than a group
    out = run.decode_cascade(0, 0, max_group=2).double().cpu().numpy()
    assert np.isnan(out[:3]).all()
    check(out[3:5], expect[3:5], "group 1")
    torch.cuda.synchronize()


@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 64), (16, 2, 256), (16, 16, 128), (64, 4, 128), (12, 4, 64)])
def test_head_shapes(hq, hkv, d):
    announce(f"read-once decode, Hq={hq} Hkv={hkv} d={d}, two groups and a singleton")
    wl = fork_workload([(96, [0, 5, 40]), (33, [0]), (300, [17, 1])], hq=hq, hkv=hkv, d=d, seed=67)
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref, fill=-1).run()
    gs, sb = run.pool.shared_prefix_plan(run.decodes[0]["seq_ids"])
    assert list(gs) == [0, 3, 4, 6] and list(sb) == [6, 0, 18]
    out = run.decode_cascade(0, 0).double().cpu().numpy()
    check(out, ref.attention(0, 0), f"Hq={hq} Hkv={hkv} d={d}")


def test_timing_events_leave_results_unchanged():
    announce("kv_timing_events on the cascade (16 x 8448 sharing 6144): outputs bit-identical, prefix time <= call time")
    wl = workloads.shared_prefix()
    run = GpuRun(wl).run()
    plain = run.decode_cascade(0, 0)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        evs = tuple(torch.cuda.Event(enable_timing=True) for _ in range(3))
        for e in evs:
            e.record(stream)
        got = run.decode_cascade(0, 0, opts=B.attention_options(timing=evs))
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int32), plain.view(torch.int32))
        k_ms, c_ms = evs[0].elapsed_time(evs[1]), evs[0].elapsed_time(evs[2])
        print(f"  preparation + prefix {k_ms * 1e3:.1f} us, call {c_ms * 1e3:.1f} us", flush=True)
        assert 0.0 < k_ms <= c_ms


# ---- quantised pools (q8_0 / q4_0): the read-once kernel with raw tiles ----

@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
@pytest.mark.parametrize("partition", [0, 64, 512])
def test_quantised_ragged_groups(fmt, partition):
    announce(f"{fmt}: ragged fork groups, empty suffixes and singletons, partition {partition}, NaN background")
    groups = [(32, [0, 0, 5]), (100, [1, 17, 300, 0]), (7, [20]), (512, [16, 16, 16, 16, 33, 1000]), (48, [0])]
    wl = replace(fork_workload(groups), kv_format=fmt)
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref, fill=-1).run()
    out = run.decode_cascade(0, 0, opts=B.attention_options(partition_tokens=partition)).double().cpu().numpy()
    check(out, ref.attention(0, 0), f"{fmt} ragged groups P={partition}")
    plain = run.decode_outputs[0][0].double().cpu().numpy()
    assert np.abs(out - plain).max() <= 2 * BF16_ABS, "read-once and plain decode of the same pool"


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
def test_quantised_shared_prefix_16x8448_full(fmt):
    announce(f"{fmt}: 16 x 8448 tokens sharing 6144, read-once decode vs oracle")
    wl = replace(workloads.shared_prefix(), kv_format=fmt)
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref).run()
    out = run.decode_cascade(0, 0).double().cpu().numpy()
    check(out, ref.attention(0, 0), f"{fmt} 16 x 8448")


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 64), (16, 2, 256), (64, 4, 128)])
def test_quantised_head_shapes(fmt, hq, hkv, d):
    announce(f"{fmt}: read-once decode, Hq={hq} Hkv={hkv} d={d}, two groups and a singleton")
    wl = replace(fork_workload([(96, [0, 5, 40]), (33, [0]), (300, [17, 1])], hq=hq, hkv=hkv, d=d, seed=67),
                 kv_format=fmt)
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref, fill=-1).run()
    out = run.decode_cascade(0, 0).double().cpu().numpy()
    check(out, ref.attention(0, 0), f"{fmt} Hq={hq} Hkv={hkv} d={d}")


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
def test_quantised_mismatched_member_gives_nan_row(fmt):
    announce(f"{fmt}: a member whose shared table entry differs gets a NaN row, the others are exact")
    wl = replace(fork_workload([(64, [0, 3, 20]), (80, [2, 2])]), kv_format=fmt)
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref, fill=-1).run()
    rec = run.decodes[0]
    expect = ref.attention(0, 0)
    tables = rec["tables"].copy()
    tables[2, 0] = tables[2, 1]
    out = run.decode_cascade(0, 0, tables=tables).double().cpu().numpy()
    assert np.isnan(out[2]).all()
    check(out[[0, 1, 3, 4]], expect[[0, 1, 3, 4]], f"{fmt} other members")
    torch.cuda.synchronize()
