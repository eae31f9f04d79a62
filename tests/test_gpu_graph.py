"""The device entry points inside a captured HIP graph.

reshape_and_cache and paged_attention_decode allocate nothing, never
synchronise and launch only kernels on the caller's stream, so a decode step
can be captured once and replayed.  The graph holds a step of one layer (the
scatter of the step's new rows, then the attention); it is replayed several
times with eager work between replays and new queries copied into its input
buffer, and every replay must equal the same step run eagerly: bit for bit on
the matrix-core kernel, within one bf16 rounding on the generic kernel (whose
waves add their outputs with LDS atomics, in any order); the eager step is
also checked against the float64 oracle.
"""

import numpy as np
import pytest
import torch

from oracle.runner import OracleReplay
from pagedattention_decode_amd import binding as B
from synth import draws, workloads
from synth.draws import TAG_K, TAG_V
from tests.gpu_harness import GpuRun, attention_errors, bits_to_float_tensor, to_device_bits

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"\n[case] {msg}", flush=True)


@pytest.mark.parametrize("kernel", [B.KV_KERNEL_MFMA, B.KV_KERNEL_GENERIC])
def test_decode_step_replays_in_a_graph(kernel):
    announce(f"reshape_and_cache + paged_attention_decode captured in a graph (kernel {kernel}), 4 replays")
    lengths = [2303, 16, 999, 4095, 33]
    seqs = tuple(range(len(lengths)))
    ops = [("add", s) for s in seqs]
    ops.append(("append", seqs, tuple(lengths)))
    ops.append(("append", seqs, tuple(1 for _ in seqs)))  # the step's own token
    ops.append(("decode", seqs))
    blocks = sum(-(-(n + 1) // 16) for n in lengths) + 8
    wl = workloads.Workload("graph_step", 81, draws.BF16, 1, 32, 8, 128, 16, blocks, ops)
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref).run()
    rec = run.decodes[0]
    n = len(seqs)
    tables = torch.from_numpy(rec["tables"]).cuda()
    lens = torch.from_numpy(rec["lengths"]).cuda()
    # the step's own token: its slots and rows (already in the pool; writing them again is the
    # same bytes, so replays of the scatter leave the pool unchanged)
    slots = torch.tensor([int(rec["tables"][i][(rec["lengths"][i] - 1) // 16]) * 16 + (rec["lengths"][i] - 1) % 16
                          for i in range(n)], dtype=torch.int64, device="cuda")
    pos = [np.array([rec["lengths"][i] - 1]) for i in range(n)]
    k_new = to_device_bits(np.concatenate([run.rows(TAG_K, 0, s, pos[i]) for i, s in enumerate(seqs)]))
    v_new = to_device_bits(np.concatenate([run.rows(TAG_V, 0, s, pos[i]) for i, s in enumerate(seqs)]))
    opts = B.attention_options(kernel=kernel)
    ws = torch.empty(max(run.pool.workspace_bytes(n, 32, tables.shape[1], opts), 1), dtype=torch.uint8,
                     device="cuda")
    q_static = to_device_bits(run.query_bits(0, 0, n))
    out_static = torch.empty_like(q_static)

    def step(q, out):
        run.pool.cache(0, k_new, v_new, slots)
        run.pool.decode(0, q, out, tables, lens, 32, opts, ws)

    step(q_static, out_static)  # eager, also warms up the library's device queries
    torch.cuda.synchronize()
    eager0 = out_static.clone()
    got = bits_to_float_tensor(eager0, wl.dtype).double().cpu().numpy()
    max_abs, rel = attention_errors(got, ref.attention(0, 0))
    print(f"  eager vs oracle: max abs {max_abs:.3e}, max row rel-L2 {rel:.3e}", flush=True)
    assert max_abs <= 2e-2 and rel <= 5e-3

    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            step(q_static, out_static)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()

    rng = np.random.default_rng(5)
    for rep in range(4):
        q_new = torch.from_numpy(rng.standard_normal((n, 32, 128), dtype=np.float32)).cuda().bfloat16()
        q_bits = q_new.view(torch.int16) if rep else q_static.clone()
        q_static.copy_(q_bits)
        out_static.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        replayed = out_static.clone()
        _ = torch.ones(1 << 20, device="cuda").sum()  # eager work between replays
        eager = torch.empty_like(q_static)
        step(q_bits, eager)
        torch.cuda.synchronize()
        if kernel == B.KV_KERNEL_MFMA:  # no atomics: the same bits every run
            assert torch.equal(replayed, eager), f"replay {rep} differs from the eager step"
            if rep == 0:
                assert torch.equal(replayed, eager0)
        else:  # the generic kernel adds its waves' outputs with LDS atomics, in any order
            a = bits_to_float_tensor(replayed, wl.dtype)
            b = bits_to_float_tensor(eager, wl.dtype)
            assert torch.isfinite(a).all()
            assert ((a - b).abs() <= 2.0 ** -7 * b.abs() + 1e-6).all(), f"replay {rep} differs from the eager step"
        print(f"  replay {rep}: equal to the eager step", flush=True)
