"""GPU parity: the HIP library against the CPU oracle.

* slot scatter (reshape_and_cache) and copy-on-write block copies: bit-exact
  against the oracle's logical pool, with every unwritten element unchanged;
* decode attention: fp32 within 1e-5 (max abs); bf16 within max abs 2e-2 and a
  per-row relative L2 error of 5e-3 against the float64 oracle;
* the workloads at their full sizes: the 12 x 131072 workload on every sequence,
  the fork workload over all 512 steps of its 36-layer pool with sampled
  (step, layer, sequence) points; ragged lengths, edge cases and both kernels.

Every test prints the case it runs before touching the GPU.
"""

import math

import numpy as np
import pytest
import torch

from oracle.attention import decode_attention
from oracle.runner import OracleReplay
from pagedattention_decode_amd import binding as B
from synth import draws, workloads
from tests import oracle_pool
from tests.gpu_harness import GpuRun, attention_errors, bits_to_float_tensor, to_device_bits

pytestmark = pytest.mark.gpu

BF16_ABS, BF16_REL, F32_ABS = 2e-2, 5e-3, 1e-5


def announce(msg):
    print(f"\n[case] {msg}", flush=True)


def check_outputs(got, expect, dtype, what):
    max_abs, rel = attention_errors(got, expect)
    print(f"  {what}: max abs {max_abs:.3e}, max row rel-L2 {rel:.3e}", flush=True)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    if dtype == draws.F32:
        assert max_abs <= F32_ABS, what
    else:
        assert max_abs <= BF16_ABS and rel <= BF16_REL, what


# ---------------------------------------------------------------------------
# pool layout decoding (independent restatement of the documented index map)
# ---------------------------------------------------------------------------

def layout_index(num_blocks, block_size, num_kv_heads, head_dim, dtype, which):
    """Flat element index of [N][B][Hkv][d] (one layer) in the device buffer."""
    X = 16 // (4 if dtype == draws.F32 else 2)
    Q = math.gcd(block_size, 4)
    p = np.arange(num_blocks)[:, None, None, None]
    r = np.arange(block_size)[None, :, None, None]
    g = np.arange(num_kv_heads)[None, None, :, None]
    e = np.arange(head_dim)[None, None, None, :]
    tile = (p * num_kv_heads + g) * block_size * head_dim
    if which == "k":
        inner = ((e // X) * block_size + r) * X + e % X
    else:
        inner = ((((e // 32) * (block_size // Q) + r // Q) * 16 + e % 16) * 2 + (e % 32) // 16) * Q + r % Q
    return tile + inner


def device_pool_logical(run: GpuRun, which, layer):
    wl = run.wl
    raw = run.pool.raw(which).cpu().numpy().view(draws.storage_np_dtype(wl.dtype))
    per_layer = wl.num_blocks * wl.block_size * wl.num_kv_heads * wl.head_dim
    idx = layout_index(wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim, wl.dtype, which)
    return raw[layer * per_layer:(layer + 1) * per_layer][idx]


# ---------------------------------------------------------------------------
# scatter and copy: bit-exact
# ---------------------------------------------------------------------------

def small_fork_workload(dtype, block_size, head_dim, num_kv_heads=2, layers=2, num_blocks=48, seed=21):
    ops = [("add", 0), ("append", (0,), (3 * block_size + 1,)), ("add", 1),
           ("append", (1, 0), (5, 2)), ("fork", 0, 2), ("fork", 0, 3),
           ("append", (2, 3, 0, 1), (1, 2, 1, block_size)), ("decode", (0, 1, 2, 3)),
           ("append", (2, 3), (block_size + 3, 1)), ("decode", (0, 1, 2, 3))]
    return workloads.Workload("small_fork", seed, dtype, layers, num_kv_heads * 2, num_kv_heads, head_dim,
                              block_size, num_blocks, ops)


@pytest.mark.parametrize("dtype,block_size,head_dim", [(draws.BF16, 16, 128), (draws.F32, 4, 64),
                                                       (draws.BF16, 2, 32), (draws.F32, 6, 96)])
def test_scatter_and_copy_bit_exact(dtype, block_size, head_dim):
    announce(f"reshape_and_cache + copy_blocks bitwise: {dtype} B={block_size} d={head_dim}")
    wl = small_fork_workload(dtype, block_size, head_dim)
    fill = 0x5A5A if dtype == draws.BF16 else 0x5A5A5A5A
    bg_val = np.array(fill, dtype=draws.storage_np_dtype(dtype))
    bg = lambda layer, which, block: np.full((block_size, 2, head_dim), bg_val)  # noqa: E731
    ref = OracleReplay(wl, background=bg).run()
    run = GpuRun(wl, fill=fill if dtype == draws.F32 else np.int16(fill), ref=ref).run()
    assert any(len(p) for _, _, _, p in ref.appends), "the workload must exercise copy-on-write"
    for layer in range(wl.num_layers):
        for which in "kv":
            dev = device_pool_logical(run, which, layer)
            expect = np.stack([ref.store.block(which, layer, p) for p in range(wl.num_blocks)])
            assert np.array_equal(dev, expect), f"{which} pool of layer {layer} differs"


def test_negative_and_out_of_range_slots_are_skipped():
    announce("reshape_and_cache skips slots < 0 and >= N*B")
    wl = small_fork_workload(draws.BF16, 16, 128, num_blocks=8)
    run = GpuRun(wl, fill=np.int16(0x1111))
    before = run.pool.raw("k").clone()
    n = 4
    k = torch.full((n, 2, 128), 7, dtype=torch.int16, device="cuda")
    slots = torch.tensor([-1, 8 * 16, 8 * 16 + 5, -100], dtype=torch.int64, device="cuda")
    run.pool.cache(0, k, k, slots)
    torch.cuda.synchronize()
    assert torch.equal(before, run.pool.raw("k"))


# ---------------------------------------------------------------------------
# attention on the workloads
# ---------------------------------------------------------------------------

def compare_all_decodes(run, ref, layers=None):
    wl = run.wl
    for i in range(len(ref.decodes)):
        for layer in (layers or range(wl.num_layers)):
            got = run.decode_outputs[i][layer].double().cpu().numpy()
            check_outputs(got, ref.attention(i, layer), wl.dtype, f"decode {i} layer {layer}")


def test_tiny_fp32_5_7_9():
    announce("tiny fp32, B=4, lengths 5/7/9, generic kernel, NaN background")
    wl = workloads.tiny_fp32()
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref, fill=-1).run()  # 0xFFFFFFFF is a NaN: unwritten slots must never count
    compare_all_decodes(run, ref)


# (the matrix-core kernel reads bf16 and quantised pools, not f32 ones)
@pytest.mark.parametrize("dtype,kernel", [(draws.BF16, B.KV_KERNEL_GENERIC), (draws.BF16, B.KV_KERNEL_MFMA),
                                          (draws.F32, B.KV_KERNEL_GENERIC)])
def test_small_fork_workload(dtype, kernel):
    announce(f"small fork workload with CoW: {dtype}, kernel {kernel}")
    wl = small_fork_workload(dtype, 16, 128)
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref, fill=-1, opts=B.attention_options(kernel=kernel)).run()
    compare_all_decodes(run, ref)


def ragged_workload(hq, hkv, d, lengths, seed=31, num_blocks=None, dtype=draws.BF16, layers=1):
    seqs = tuple(range(len(lengths)))
    ops = [("add", s) for s in seqs]
    ops.append(("append", seqs, tuple(lengths)))
    ops.append(("decode", seqs))
    need = sum(-(-n // 16) for n in lengths)
    return workloads.Workload("ragged", seed, dtype, layers, hq, hkv, d, 16, num_blocks or need + 7, ops)


RAGGED = [1, 2, 15, 16, 17, 31, 100, 257, 511, 512, 513, 1000, 2049]


@pytest.mark.parametrize("kernel", [B.KV_KERNEL_MFMA, B.KV_KERNEL_GENERIC])
@pytest.mark.parametrize("partition", [0, 16, 48, 256, 512, 1024, 4096])
def test_ragged_lengths_and_partitions(kernel, partition):
    announce(f"ragged lengths {RAGGED}, kernel {kernel}, partition {partition}")
    wl = ragged_workload(32, 8, 128, RAGGED)
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref, fill=-1,
                 opts=B.attention_options(partition_tokens=partition, kernel=kernel)).run()
    compare_all_decodes(run, ref)


@pytest.mark.parametrize("hq,hkv,d", [(8, 8, 128), (64, 8, 128), (48, 3, 128), (16, 1, 128),
                                      (32, 8, 64), (16, 4, 256), (12, 4, 64)])
def test_head_shapes(hq, hkv, d):
    announce(f"head shapes Hq={hq} Hkv={hkv} d={d}, both kernels")
    wl = ragged_workload(hq, hkv, d, [1, 7, 16, 33, 300, 700])
    ref = OracleReplay(wl).run()
    for kernel in (B.KV_KERNEL_MFMA, B.KV_KERNEL_GENERIC):
        run = GpuRun(wl, ref=ref, fill=-1, opts=B.attention_options(partition_tokens=128, kernel=kernel)).run()
        compare_all_decodes(run, ref)


def test_qwen3_8b_37x2304_full():
    announce("Qwen3-8B-shaped layer, 37 x 2304 tokens, bf16, default launch")
    wl = workloads.qwen_independent()
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref).run()
    compare_all_decodes(run, ref)


def test_shared_prefix_16x8448_full():
    announce("16 x 8448 tokens sharing 6144, bf16, default launch")
    wl = workloads.shared_prefix()
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref).run()
    compare_all_decodes(run, ref)
    # forks share before divergence: the prefix blocks of all 16 tables coincide
    tables = run.decodes[0]["tables"]
    assert (tables[:, :384] == tables[0, :384]).all()


@pytest.mark.timeout(1800)
def test_gqa70b_12x131072_full():
    announce("70B-GQA layer, 12 x 131072 tokens, Hq=64: every sequence written and compared, split-K 512 "
             "(the benchmarked launch) and the automatic partition")
    wl = workloads.gqa70b_128k()
    S = 12
    # the oracle's outputs: one process per sequence, each writing that sequence's K/V only
    res = oracle_pool.evaluate([("gqa70b_128k", {}, [0], [s], [(0, 0, [s])]) for s in range(S)])
    expect = np.concatenate([r[0] for r in res])
    # slots and tables of the whole batch are checked against the oracle's block manager
    ref = OracleReplay(wl, layers=[], writers=set()).run()
    run = GpuRun(wl, ref=ref, opts=B.attention_options(partition_tokens=512)).run()
    got = run.decode_outputs[0][0].double().cpu().numpy()
    for s in range(S):
        check_outputs(got[s:s + 1], expect[s:s + 1], wl.dtype, f"sequence {s}, split-K 512")
    rec = run.decodes[0]
    d_tables = torch.from_numpy(rec["tables"]).cuda()
    d_lens = torch.from_numpy(rec["lengths"]).cuda()
    auto = run.decode(0, 0, d_tables, d_lens, S, opts=B.attention_options()).double().cpu().numpy()
    check_outputs(auto, expect, wl.dtype, "all sequences, automatic partition")


# the fork workload's sampled steps, layers and sequences: the first copy-on-write
# step, the first block crossings of the divergent suffixes (steps 15 / 16), the
# middle and the last step; the first, middle and last layer of the 36-layer pool;
# sequences of every root, roots and forks
FORK_STEPS = (0, 1, 15, 16, 255, 511)
FORK_LAYERS = (0, 17, 35)
FORK_ROWS = (0, 1, 15, 16, 47, 63)
FORK_ROOT_OF = {0: 0, 1: 0, 15: 0, 16: 16, 47: 32, 63: 48}


def fork_oracle():
    """{(step, layer, sequence): [Hq, d]} of the oracle on the sampled points, replayed
    per (layer, root) in parallel processes."""
    by_root = {}
    for r in FORK_ROWS:
        by_root.setdefault(FORK_ROOT_OF[r], []).append(r)
    tasks = []
    for layer in FORK_LAYERS:
        for root, rows in by_root.items():
            step_sets = (FORK_STEPS[:3], FORK_STEPS[3:]) if len(rows) > 1 else (FORK_STEPS,)
            for steps in step_sets:
                tasks.append(("agentic_fork", {"steps": 512, "layers": 36}, [layer], sorted(set(rows) | {root}),
                              [(i, layer, rows) for i in steps]))
    expect = {}
    for task, outs in zip(tasks, oracle_pool.evaluate(tasks)):
        for (i, layer, rows), out in zip(task[4], outs):
            for r, o in zip(rows, out):
                expect[(i, layer, r)] = o
    return expect


@pytest.mark.timeout(1800)
def test_agentic_fork_sampled():
    announce("fork workload: 4 roots x 32769, 16 forks each, all 512 steps over the 36-layer pool; plain and "
             f"read-once decode at steps {FORK_STEPS} x layers {FORK_LAYERS}, sequences {FORK_ROWS}")
    wl = workloads.agentic_fork(steps=512, layers=36)
    expect = fork_oracle()
    writers = set(FORK_ROWS) | set(FORK_ROOT_OF.values())
    ref = OracleReplay(wl, layers=[], writers=set()).run()  # slots, copy pairs and tables, bit for bit
    run = GpuRun(wl, ref=ref, layers=list(FORK_LAYERS), writers=writers, decode_steps=FORK_STEPS).run()
    assert sum(len(p) for _, p in run.appends) == 60, "60 copy-on-write copies at the first divergent step"
    rows = list(FORK_ROWS)
    for i in FORK_STEPS:
        gs, sb = run.pool.shared_prefix_plan(run.decodes[i]["seq_ids"])
        assert len(sb) == 4 and all(b == 2048 for b in sb), (list(gs), list(sb))
        for layer in FORK_LAYERS:
            exp = np.stack([expect[(i, layer, r)] for r in rows])
            got = run.decode_outputs[i][layer].double().cpu().numpy()[rows]
            check_outputs(got, exp, wl.dtype, f"step {i} layer {layer}")
            got = run.decode_cascade(i, layer).double().cpu().numpy()[rows]
            check_outputs(got, exp, wl.dtype, f"step {i} layer {layer}, read-once decode")


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------

def test_zero_length_context_gives_zero_row_and_bad_entry_gives_nan():
    announce("context_len 0 -> zero row; out-of-range table entry -> NaN row; empty batch")
    wl = ragged_workload(32, 8, 128, [40, 40, 40])
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref, fill=-1).run()
    tables = torch.from_numpy(run.decodes[0]["tables"]).cuda()
    lens = torch.from_numpy(run.decodes[0]["lengths"]).cuda()
    lens[1] = 0
    tables[2, 1] = wl.num_blocks + 5
    for kernel in (B.KV_KERNEL_MFMA, B.KV_KERNEL_GENERIC):
        for part in (16, 0):
            out = run.decode(0, 0, tables, lens, 3, opts=B.attention_options(partition_tokens=part, kernel=kernel))
            o = out.double().cpu().numpy()
            check_outputs(o[:1], ref.attention(0, 0, rows=[0]), wl.dtype, "row 0 unaffected")
            assert (o[1] == 0).all()
            assert np.isnan(o[2]).all()
    # an empty batch is a no-op
    empty_t = torch.zeros((0, 4), dtype=torch.int32, device="cuda")
    empty_l = torch.zeros((0,), dtype=torch.int32, device="cuda")
    q = torch.zeros((0, 32, 128), dtype=torch.int16, device="cuda")
    run.pool.decode(0, q, q.clone(), empty_t, empty_l, 32)
    torch.cuda.synchronize()


def test_single_token_context_returns_its_value():
    announce("n = 1: the output equals v_0 rounded to bf16")
    wl = ragged_workload(32, 8, 128, [1, 1])
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref, fill=-1).run()
    got = run.decode_outputs[0][0].cpu().numpy()
    for s in range(2):
        _, vb = ref.store.gather(0, ref.decodes[0]["tables"][s], 1)
        v = draws.bits_to_f64(vb, wl.dtype)[0]  # [Hkv, d]
        expect = np.repeat(v, 4, axis=0)
        assert np.array_equal(got[s].astype(np.float64), expect)


def test_split_and_single_pass_agree():
    announce("split-K partitions vs one partition vs generic kernel on 2049 tokens")
    wl = ragged_workload(32, 8, 128, [2049, 1500])
    ref = OracleReplay(wl).run()
    outs = []
    for kernel, part in ((B.KV_KERNEL_GENERIC, 4096), (B.KV_KERNEL_MFMA, 4096), (B.KV_KERNEL_MFMA, 64),
                         (B.KV_KERNEL_MFMA, 16), (B.KV_KERNEL_GENERIC, 32)):
        run = GpuRun(wl, ref=ref, opts=B.attention_options(partition_tokens=part, kernel=kernel)).run()
        outs.append(run.decode_outputs[0][0].double().cpu().numpy())
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() <= 2 * BF16_ABS



@pytest.mark.parametrize("kernel", [B.KV_KERNEL_GENERIC, B.KV_KERNEL_MFMA])
def test_repeated_calls_give_identical_bits(kernel):
    announce(f"kernel {kernel}: five calls on one input give the same output bits")
    wl = ragged_workload(32, 8, 128, [2049, 700, 33, 1, 1500], layers=1)
    run = GpuRun(wl).run()
    tables = torch.from_numpy(run.decodes[0]["tables"]).cuda()
    lens = torch.from_numpy(run.decodes[0]["lengths"]).cuda()
    outs = [run.decode(0, 0, tables, lens, 5, opts=B.attention_options(kernel=kernel, partition_tokens=256))
            for _ in range(5)]
    for o in outs[1:]:
        assert torch.equal(o, outs[0]), "the output bits changed between calls"


def test_workspace_reused_across_calls():
    announce("split-K kernel: one workspace reused by 6 calls (layers 0, 1 alternating), outputs poisoned")
    lengths = [2304, 17, 1000, 4096, 33, 2304, 700, 1]
    wl = ragged_workload(32, 8, 128, lengths, layers=2)
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref, fill=-1).run()
    tables = torch.from_numpy(run.decodes[0]["tables"]).cuda()
    lens = torch.from_numpy(run.decodes[0]["lengths"]).cuda()
    n = len(lengths)
    opts = B.attention_options(kernel=B.KV_KERNEL_MFMA)
    ws = torch.empty(run.pool.workspace_bytes(n, 32, tables.shape[1], opts), dtype=torch.uint8, device="cuda")
    ws.fill_(0xFF)
    out = torch.empty((n, 32, 128), dtype=torch.int16, device="cuda")
    for call in range(6):
        layer = call % 2
        q = to_device_bits(run.query_bits(0, layer, n))
        out.fill_(-1)
        run.pool.decode(layer, q, out, tables, lens, 32, opts, ws)
        got = bits_to_float_tensor(out, wl.dtype).double().cpu().numpy()
        check_outputs(got, ref.attention(0, layer), wl.dtype, f"call {call} layer {layer}")


def test_invalid_arguments_are_rejected():
    announce("argument validation of the device entry points")
    wl = ragged_workload(32, 8, 128, [20])
    run = GpuRun(wl).run()
    t = torch.from_numpy(run.decodes[0]["tables"]).cuda()
    l_ = torch.from_numpy(run.decodes[0]["lengths"]).cuda()
    q = torch.zeros((1, 32, 128), dtype=torch.int16, device="cuda")
    with pytest.raises(B.KVError):
        run.pool.decode(0, q, q.clone(), t, l_, 30)  # Hq not a multiple of Hkv
    with pytest.raises(B.KVError):
        run.pool.decode(3, q, q.clone(), t, l_, 32)  # layer out of range
    with pytest.raises(B.KVError):
        run.pool.decode(0, q, q.clone(), t, l_, 32, opts=B.attention_options(partition_tokens=24))
    with pytest.raises(B.KVError):  # needs a workspace
        run.pool.decode(0, q, q.clone(), t, l_, 32, opts=B.attention_options(partition_tokens=16))
    with pytest.raises(B.KVError):
        run.pool.decode(0, q, q.clone(), t, l_, 8 * 17)  # G = 17
    # the binding refuses tensors of the wrong element type, shape or device before the call
    slots32 = torch.zeros((1,), dtype=torch.int32, device="cuda")
    row = torch.zeros((1, 8, 128), dtype=torch.int16, device="cuda")
    bad_calls = {
        "int32 slot mapping": lambda: run.pool.cache(0, row, row, slots32),
        "k rows of 4-byte elements": lambda: run.pool.cache(0, row.float(), row, slots32.long()),
        "k rows of the wrong head count": lambda: run.pool.cache(0, row[:, :4].contiguous(), row, slots32.long()),
        "int64 block tables": lambda: run.pool.decode(0, q, q.clone(), t.long(), l_, 32),
        "int64 context lengths": lambda: run.pool.decode(0, q, q.clone(), t, l_.long(), 32),
        "float32 queries on a bf16 pool": lambda: run.pool.decode(0, q.float(), q.clone(), t, l_, 32),
        "queries of the wrong head dim": lambda: run.pool.decode(0, q[:, :, :64].contiguous(), q.clone(), t, l_, 32),
        "host queries": lambda: run.pool.decode(0, q.cpu(), q.clone(), t, l_, 32),
        "lengths of another batch": lambda: run.pool.decode(0, q, q.clone(), t, torch.cat([l_, l_]), 32),
        "int32 copy pairs": lambda: run.pool.copy(torch.zeros((1, 2), dtype=torch.int32, device="cuda")),
    }
    for what, call in bad_calls.items():
        with pytest.raises(B.KVArgumentError):
            call()
        print(f"  refused: {what}", flush=True)
    f32 = small_fork_workload(draws.F32, 4, 64)
    r2 = GpuRun(f32)
    with pytest.raises(B.KVError) as e:
        r2.pool.decode(0, torch.zeros((1, 4, 64), dtype=torch.int32, device="cuda"),
                       torch.zeros((1, 4, 64), dtype=torch.int32, device="cuda"),
                       torch.zeros((1, 2), dtype=torch.int32, device="cuda"),
                       torch.ones((1,), dtype=torch.int32, device="cuda"), 4,
                       opts=B.attention_options(kernel=B.KV_KERNEL_MFMA))
    assert e.value.status == B.KV_ERR_UNSUPPORTED


def test_release_waits_for_stream_event():
    announce("kv_seq_release defers reuse until the stream's work completes")
    wl = ragged_workload(32, 8, 128, [64, 64], num_blocks=8)
    run = GpuRun(wl).run()
    stream = torch.cuda.current_stream()
    run.pool.release(0, stream)
    st = run.pool.stats()
    assert st["n_pending"] + st["n_free"] == 4 and st["n_allocated"] == 4
    run.pool.reclaim(wait=True)
    st = run.pool.stats()
    assert st["n_pending"] == 0 and st["n_free"] == 4
    run.pool.check()


@pytest.mark.parametrize("kernel", [B.KV_KERNEL_MFMA, B.KV_KERNEL_GENERIC])
def test_timing_events_leave_results_unchanged(kernel):
    announce(f"kv_timing_events on decode calls (kernel {kernel}): outputs as without them, times ordered")
    lengths = [2304, 17, 1000, 33]
    wl = ragged_workload(32, 8, 128, lengths)
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref).run()
    tables = torch.from_numpy(run.decodes[0]["tables"]).cuda()
    lens = torch.from_numpy(run.decodes[0]["lengths"]).cuda()
    n = len(lengths)
    stream = torch.cuda.current_stream()
    q = to_device_bits(run.query_bits(0, 0, n))
    plain = B.attention_options(kernel=kernel)
    ws = torch.empty(max(run.pool.workspace_bytes(n, 32, tables.shape[1], plain), 1), dtype=torch.uint8,
                     device="cuda")
    out0 = torch.empty((n, 32, 128), dtype=torch.int16, device="cuda")
    run.pool.decode(0, q, out0, tables, lens, 32, plain, ws)
    for _ in range(3):
        evs = tuple(torch.cuda.Event(enable_timing=True) for _ in range(3))
        for e in evs:
            e.record(stream)
        out = torch.full((n, 32, 128), -1, dtype=torch.int16, device="cuda")
        run.pool.decode(0, q, out, tables, lens, 32, B.attention_options(kernel=kernel, timing=evs), ws)
        torch.cuda.synchronize()
        assert torch.equal(out, out0)
        k_ms, c_ms = evs[0].elapsed_time(evs[1]), evs[0].elapsed_time(evs[2])
        print(f"  kernel {k_ms * 1e3:.1f} us, call {c_ms * 1e3:.1f} us", flush=True)
        assert 0.0 < k_ms <= c_ms
    got = bits_to_float_tensor(out0, wl.dtype).double().cpu().numpy()
    check_outputs(got, ref.attention(0, 0), wl.dtype, "decode")


def test_more_sequences_than_one_launch_takes():
    announce("5000 sequences (more than the 4095 one split-K launch takes), Hq=8 Hkv=2 d=64, lengths 1..40: "
             "consecutive launches, automatic and matrix-core selection")
    rng = np.random.default_rng(77)
    lengths = [int(x) for x in rng.integers(1, 41, size=5000)]
    wl = ragged_workload(8, 2, 64, lengths, seed=41)
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref, fill=-1, opts=B.attention_options(kernel=B.KV_KERNEL_MFMA)).run()
    compare_all_decodes(run, ref)
    rec = run.decodes[0]
    tables = torch.from_numpy(rec["tables"]).cuda()
    lens = torch.from_numpy(rec["lengths"]).cuda()
    auto = run.decode(0, 0, tables, lens, len(lengths), opts=B.attention_options())
    mfma = run.decode(0, 0, tables, lens, len(lengths), opts=B.attention_options(kernel=B.KV_KERNEL_MFMA))
    assert torch.equal(auto, mfma), "the automatic choice is not the matrix-core kernel above 4095 sequences"
