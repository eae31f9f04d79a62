"""GPU parity of the host tier (swap of blocks to pinned host frames and back).

* swap-out: every frame holds, byte for byte, the oracle's block in the
  documented frame layout (bf16 pools start from a known background, so whole
  frames compare; quantised pools compare the live slots' codes and scales);
* swap-in: the new blocks hold the oracle's block bytes again, and every
  decode (before, between and after the swaps, while other sequences reuse the
  freed blocks) matches the oracle's attention at the bf16 bar;
* the pairs of every swap equal the oracle's (checked by the harness).
Cases: shuffled and consecutive frames, a staging buffer smaller than a swap
(several chunks), q8_0 and q4_0 pools, a separate copy stream.
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle.runner import OracleReplay
from synth import draws, workloads
from tests.gpu_harness import GpuRun, attention_errors
from tests.test_gpu_parity import device_pool_logical, layout_index
from tests.test_gpu_quant import decode_tiles

pytestmark = pytest.mark.gpu

BF16_ABS, BF16_REL = 2e-2, 5e-3
BACKGROUND = 0xFFFF  # bf16 NaN bits in every slot nobody wrote


def announce(msg):
    print(f"\n[case] {msg}", flush=True)


def check(got, expect, what):
    max_abs, rel = attention_errors(got, expect)
    print(f"  {what}: max abs {max_abs:.3e}, max row rel-L2 {rel:.3e}", flush=True)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert max_abs <= BF16_ABS and rel <= BF16_REL, what


def background(wl):
    return lambda layer, which, block: np.full((wl.block_size, wl.num_kv_heads, wl.head_dim), BACKGROUND, np.uint16)


def frame_chunk(run, frame, layer, which):
    """Bytes of one layer's K or V tiles inside a host frame (documented frame layout)."""
    F = run.pool.frame_bytes
    chunk = F // (2 * run.wl.num_layers)
    raw = run.pool.host_frames.numpy()[frame * F:(frame + 1) * F]
    off = (2 * layer + (1 if which == "v" else 0)) * chunk
    return raw[off:off + chunk]


def bf16_frame_checker(ref):
    def on_swap(run, i):
        wl = run.wl
        kind, seq, pairs = run.swaps[i]
        rec = ref.swaps[i]
        if kind != "swap_out":
            return
        # the oracle state after the whole workload still holds every frame written by its
        # last swap-out unless a later swap-out reused it; compare against the record's copy
        for block, frame in pairs.tolist():
            for layer in range(wl.num_layers):
                for which in ("k", "v"):
                    elems = frame_chunk(run, frame, layer, which).view(np.uint16)
                    idx = layout_index(1, wl.block_size, wl.num_kv_heads, wl.head_dim, wl.dtype, which)
                    got = elems[idx][0]  # [B, Hkv, d]
                    expect = rec["host"][(layer, which, frame)]
                    assert np.array_equal(got, expect), f"frame {frame} layer {layer} {which}"
    return on_swap


class RecordingReplay(OracleReplay):
    """The oracle replay, keeping a copy of every frame at the moment of its swap-out."""

    def apply(self, op):
        super().apply(op)
        if op[0] == "swap_out":
            rec = self.swaps[-1]
            rec["host"] = {}
            for _, frame in rec["pairs"]:
                for layer in self.layers:
                    for which in ("k", "v"):
                        hb = self.store.host_block(which, layer, frame)
                        rec["host"][(layer, which, frame)] = \
                            tuple(x.copy() for x in hb) if isinstance(hb, tuple) else hb.copy()


def run_tool_pause(wl, **kw):
    ref = RecordingReplay(wl, background=None if wl.kv_format else background(wl), eager=True).run()
    fill = None if wl.kv_format else -1
    on_swap = None if wl.kv_format else bf16_frame_checker(ref)
    run = GpuRun(wl, ref=ref, fill=fill, on_swap=kw.pop("on_swap", on_swap), **kw).run()
    return ref, run


def check_decodes(run, ref):
    """Rows with keys against the oracle; a sequence with no token yet gives a zero row."""
    for i, rec in enumerate(ref.decodes):
        rows = [r for r, n in enumerate(rec["lengths"]) if n > 0]
        empty = [r for r, n in enumerate(rec["lengths"]) if n == 0]
        for layer in run.decode_layers:
            got = run.decode_outputs[i][layer].double().cpu().numpy()
            check(got[rows], ref.attention(i, layer, rows=rows), f"decode {i} L{layer}")
            assert np.all(got[empty] == 0)


def check_blocks_back(run, ref):
    """After every swap-in the new blocks hold the oracle's bytes (whole blocks, bf16)."""
    wl = run.wl
    last_in = {}
    for kind, seq, pairs in run.swaps:
        if kind == "swap_in":
            last_in[seq] = pairs
    for layer in range(wl.num_layers):
        for which in ("k", "v"):
            dev = device_pool_logical(run, which, layer)  # [N, B, Hkv, d]
            for seq, pairs in last_in.items():
                for frame, block in pairs.tolist():
                    # the sequence wrote one more token after coming back: compare the block as the
                    # oracle holds it at the end
                    assert np.array_equal(dev[block], ref.store.block(which, layer, block)), (seq, block)


@pytest.mark.parametrize("frames", ["shuffled", "sequential"])
def test_tool_pause_bf16(frames):
    announce(f"tool pause, bf16, {frames} host frames: frames, blocks and decodes vs the oracle")
    wl = workloads.tool_pause(frames=frames)
    ref, run = run_tool_pause(wl)
    assert len(run.swaps) == 4
    check_decodes(run, ref)
    check_blocks_back(run, ref)
    run.pool.check()


def test_tool_pause_small_staging():
    announce("tool pause, staging of 5 frames: every swap runs in chunks")
    wl = workloads.tool_pause(frames="sequential")
    frame = 2 * wl.num_layers * wl.num_kv_heads * wl.block_size * wl.head_dim * 2
    ref, run = run_tool_pause(wl, staging_bytes=5 * frame)
    assert run.pool.staging.numel() == 5 * run.pool.frame_bytes
    check_decodes(run, ref)
    check_blocks_back(run, ref)


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
def test_tool_pause_quantised(fmt):
    announce(f"tool pause, {fmt} pool: live codes and scales in the frames, decodes after the swap-in")
    wl = replace(workloads.tool_pause(), kv_format=fmt)
    seen = []

    def on_swap(run, i):
        kind, seq, pairs = run.swaps[i]
        if kind != "swap_out":
            return
        rec = ref_holder[0].swaps[i]
        for (block, frame), j in zip(pairs.tolist(), rec["positions"]):
            live = min(16, rec["length"] - 16 * j)
            for layer in range(wl.num_layers):
                for which in ("k", "v"):
                    k, v, scales = decode_tiles(frame_chunk(run, frame, layer, which), fmt, 1, wl.num_kv_heads,
                                                wl.head_dim)
                    codes = k if which == "k" else v
                    e_codes, e_scales = rec["host"][(layer, which, frame)]
                    assert np.array_equal(codes[0][:, :live], e_codes[:live].transpose(1, 0, 2))
                    assert np.array_equal(scales[0][:, :live], e_scales[:live].transpose(1, 0, 2))
            seen.append(frame)

    ref_holder = [RecordingReplay(wl, eager=True).run()]
    run = GpuRun(wl, ref=ref_holder[0], on_swap=on_swap).run()
    assert len(seen) == 145
    check_decodes(run, ref_holder[0])


def test_copy_stream():
    announce("tool pause on a separate copy stream, ordered by events")
    wl = workloads.tool_pause(layers=1)
    ref = OracleReplay(wl, eager=True).run()
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()

    class SideRun(GpuRun):
        def apply(self, op):
            if op[0] in ("swap_out", "swap_in"):
                side.wait_stream(main)  # the copy reads blocks the main stream wrote
                with torch.cuda.stream(side):
                    pairs = self.pool.swap_out(op[1], stream=side) if op[0] == "swap_out" \
                        else self.pool.swap_in(op[1], stream=side)
                main.wait_stream(side)  # later decodes read what the copy wrote
                self.pool.reclaim(True)
                r = self.ref.swaps[len(self.swaps)]
                assert [tuple(p) for p in pairs.tolist()] == [tuple(p) for p in r["pairs"]]
                self.swaps.append((op[0], op[1], pairs))
                return
            super().apply(op)

    run = SideRun(wl, ref=ref).run()
    check_decodes(run, ref)


def test_swap_round_trip_of_every_block_of_a_long_sequence():
    announce("one 4000-token sequence alone: out, the pool refilled by another, back in; bytes and decode")
    ops = [("host", 300), ("add", 0), ("append", (0,), (4000,)), ("decode", (0,)), ("swap_out", 0),
           ("add", 1), ("append", (1,), (4000,)), ("decode", (1,)), ("release", 1), ("swap_in", 0),
           ("decode", (0,))]
    wl = workloads.Workload("round_trip", 12, draws.BF16, 3, 16, 2, 128, 16, 270, ops)
    ref, run = run_tool_pause(wl)
    out = ref.decodes[0]
    back = ref.decodes[2]
    assert out["tables"][0] != back["tables"][0]  # other blocks, same values
    check_decodes(run, ref)
    check_blocks_back(run, ref)


@pytest.mark.parametrize("dtype,block,hkv,d", [(draws.F32, 4, 2, 64), (draws.BF16, 6, 1, 32), (draws.BF16, 16, 4, 256)])
def test_other_pool_shapes(dtype, block, hkv, d):
    announce(f"swap on a {dtype} pool, B={block}, Hkv={hkv}, d={d}: frames and blocks bit-exact")
    ops = [("host", 64, "sequential"), ("add", 0), ("add", 1), ("append", (0, 1), (5 * block + 1, 3 * block + 2)),
           ("fork", 1, 2), ("append", (2,), (2,)), ("swap_out", 0), ("swap_out", 1),
           ("add", 3), ("append", (3,), (7 * block,)), ("swap_in", 1), ("swap_in", 0)]
    wl = workloads.Workload("swap_shapes", 71, dtype, 2, 2 * hkv, hkv, d, block, 40, ops)
    bits = np.uint32 if dtype == draws.F32 else np.uint16
    pattern = 0xFFFFFFFF if dtype == draws.F32 else 0xFFFF

    def bg(layer, which, b):
        return np.full((block, hkv, d), pattern, bits)

    ref = RecordingReplay(wl, background=bg, eager=True).run()
    seen = []

    def on_swap(run, i):
        kind, seq, pairs = run.swaps[i]
        if kind != "swap_out":
            return
        for block_id, frame in pairs.tolist():
            for layer in range(wl.num_layers):
                for which in ("k", "v"):
                    elems = frame_chunk(run, frame, layer, which).view(bits)
                    idx = layout_index(1, block, hkv, d, dtype, which)
                    assert np.array_equal(elems[idx][0], ref.swaps[i]["host"][(layer, which, frame)])
            seen.append(frame)

    run = GpuRun(wl, ref=ref, fill=-1, on_swap=on_swap).run()
    # sequence 0 moves its 6 blocks; sequence 1 only the block its fork copied away from it,
    # the other 3 stay shared in HBM
    assert len(seen) == 6 + 1
    check_blocks_back(run, ref)
    run.pool.check()
