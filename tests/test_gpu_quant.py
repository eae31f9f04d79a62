"""GPU parity of the quantised KV cache (q8_0, q4_0) against the oracle.

* reshape_and_cache into a quantised pool: codes and scales bit-exact with the
  oracle's quantisation (both take the float32 steps the header documents),
  every byte of an unwritten slot unchanged;
* copy_blocks on a quantised pool: bitwise tile copies;
* decode attention over the quantised pool: against the oracle's float64
  attention on exactly the dequantised values, bf16 bar (max abs 2e-2, per-row
  relative L2 5e-3).

The pool bytes are decoded by an independent restatement of the documented
tile layout (include/pagedkv.h).  Every test prints its case first.
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
BITS = {"q8_0": 8, "q4_0": 4}


def announce(msg):
    print(f"\n[case] {msg}", flush=True)


def check(got, expect, what):
    max_abs, rel = attention_errors(got, expect)
    print(f"  {what}: max abs {max_abs:.3e}, max row rel-L2 {rel:.3e}", flush=True)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert max_abs <= BF16_ABS and rel <= BF16_REL, what


def decode_tiles(raw, fmt, num_blocks, hkv, d):
    """One layer's bytes -> (K codes, V codes, scales): codes int16 [N, Hkv, 16, d] read with the
    K and with the V lane order, scales uint16 [N, Hkv, 16, d/32]."""
    bits = BITS[fmt]
    cb = 16 * d * bits // 8
    tb = cb + d
    tiles = raw.reshape(num_blocks, hkv, tb)
    scales = tiles[..., cb:].copy().view(np.uint16).reshape(num_blocks, hkv, 16, d // 32)
    lb = d * bits // 32
    lanes = tiles[..., :cb].reshape(num_blocks, hkv, 64, lb)
    k = np.empty((num_blocks, hkv, 16, d), np.int16)
    v = np.empty((num_blocks, hkv, 16, d), np.int16)
    for q in range(4):
        for r in range(16):
            lane = lanes[:, :, 16 * q + r, :]
            for kk in range(d // 32):
                for j in range(8):
                    dim = 32 * kk + 8 * q + j
                    if bits == 8:
                        k[:, :, r, dim] = lane[..., 8 * kk + j].astype(np.int8)
                    else:
                        byte = lane[..., 4 * kk + j % 4]
                        nib = (byte >> 4) if j >= 4 else (byte & 0x0F)
                        k[:, :, r, dim] = nib.astype(np.int16) - 8
            # V: lane (q, r) holds dim 16 t + r of tokens 4 q + i
            for t in range(d // 16):
                for i in range(4):
                    dim = 16 * t + r
                    if bits == 8:
                        v[:, :, 4 * q + i, dim] = lane[..., 4 * t + i].astype(np.int8)
                    else:
                        byte = lane[..., 4 * (t // 2) + i]
                        nib = (byte >> 4) if t % 2 else (byte & 0x0F)
                        v[:, :, 4 * q + i, dim] = nib.astype(np.int16) - 8
    return k, v, scales


def quant_workload(fmt, hq=32, hkv=8, d=128, lengths=(1, 15, 16, 17, 100, 700), layers=2, seed=51):
    seqs = tuple(range(len(lengths)))
    ops = [("add", s) for s in seqs]
    ops.append(("append", seqs, tuple(lengths)))
    ops.append(("decode", seqs))
    blocks = sum(-(-n // 16) for n in lengths) + 5
    return workloads.Workload(f"quant_{fmt}", seed, draws.BF16, layers, hq, hkv, d, 16, blocks, ops, kv_format=fmt)


def compare_pool(run, ref, layer):
    wl = run.wl
    kb = run.pool.raw("k").cpu().numpy()
    vb = run.pool.raw("v").cpu().numpy()
    per_layer = kb.size // wl.num_layers
    sl = slice(layer * per_layer, (layer + 1) * per_layer)
    gk, _, gks = decode_tiles(kb[sl], wl.kv_format, wl.num_blocks, wl.num_kv_heads, wl.head_dim)
    _, gv, gvs = decode_tiles(vb[sl], wl.kv_format, wl.num_blocks, wl.num_kv_heads, wl.head_dim)
    # the live tokens of the last decode: every one was written, directly or by a block copy
    dec = ref.decodes[-1]
    live = {}
    for table, n in zip(dec["tables"], dec["lengths"]):
        for t in range(n):
            live.setdefault(table[t // 16], set()).add(t % 16)
    for blk, slots in live.items():
        codes, scales = ref.store.block("k", layer, blk)
        vcodes, vscales = ref.store.block("v", layer, blk)
        sl = sorted(slots)
        # oracle blocks are [slot, head, ...]; the pool's are [head, slot, ...]
        assert np.array_equal(gk[blk][:, sl], codes[sl].transpose(1, 0, 2)), f"K codes of block {blk}"
        assert np.array_equal(gks[blk][:, sl], scales[sl].transpose(1, 0, 2)), f"K scales of block {blk}"
        assert np.array_equal(gv[blk][:, sl], vcodes[sl].transpose(1, 0, 2)), f"V codes of block {blk}"
        assert np.array_equal(gvs[blk][:, sl], vscales[sl].transpose(1, 0, 2)), f"V scales of block {blk}"
    return len(live)


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_quantised_scatter_is_bit_exact(fmt, d):
    announce(f"reshape_and_cache into a {fmt} pool, d={d}: codes and scales bit-exact")
    lengths = (1, 15, 16, 17, 40)
    wl = quant_workload(fmt, hq=8, hkv=4, d=d, lengths=lengths)
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref).run()
    for layer in range(wl.num_layers):
        assert compare_pool(run, ref, layer) == sum(-(-n // 16) for n in lengths)


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
def test_unwritten_slots_keep_their_bytes(fmt):
    announce(f"{fmt}: a partly written block keeps the background bytes of its other slots")
    wl = quant_workload(fmt, hq=8, hkv=2, d=64, lengths=(5,), layers=1)
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref, fill=-1).run()
    raw = run.pool.raw("k").cpu().numpy()
    blk = ref.decodes[0]["tables"][0][0]
    gk, _, gks = decode_tiles(raw, fmt, wl.num_blocks, wl.num_kv_heads, wl.head_dim)
    codes, scales = ref.store.block("k", 0, blk)
    assert np.array_equal(gk[blk][:, :5], codes.transpose(1, 0, 2)[:, :5])
    assert np.all(gks[blk][:, 5:] == 0xFFFF)          # scales of slots 5.. untouched
    background = -1 if fmt == "q8_0" else 7            # an all-ones byte decodes to -1 / 15 - 8
    assert np.all(gk[blk][:, 5:] == background)
    other = [b for b in range(wl.num_blocks) if b != blk]
    assert np.all(gks[other] == 0xFFFF)


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
def test_copy_on_write_copies_quantised_tiles(fmt):
    announce(f"{fmt}: fork, then a divergent append copies the shared block bitwise")
    ops = [("add", 0), ("append", (0,), (21,)), ("fork", 0, 1), ("append", (1, 0), (2, 1)), ("decode", (0, 1))]
    wl = workloads.Workload(f"cow_{fmt}", 52, draws.BF16, 2, 8, 2, 128, 16, 12, ops, kv_format=fmt)
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref).run()
    assert any(len(a[3]) for a in ref.appends), "the workload must copy a block"
    for layer in range(2):
        compare_pool(run, ref, layer)
    for b in range(2):
        check(run.decode_outputs[0][0].double().cpu().numpy()[b:b + 1], ref.attention(0, 0, rows=[b]),
              f"{fmt} row {b}")


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
@pytest.mark.parametrize("partition", [0, 64, 512])
def test_quantised_decode_ragged(fmt, partition):
    announce(f"{fmt} decode, ragged lengths, partition {partition}, background NaN bytes")
    wl = quant_workload(fmt, lengths=(1, 2, 15, 16, 17, 100, 511, 513, 1000, 2049), layers=1)
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref, fill=-1, opts=B.attention_options(partition_tokens=partition)).run()
    check(run.decode_outputs[0][0].double().cpu().numpy(), ref.attention(0, 0), f"{fmt} P={partition}")


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
@pytest.mark.parametrize("hq,hkv,d", [(64, 8, 128), (16, 1, 128), (32, 8, 64), (16, 4, 256), (12, 4, 64)])
def test_quantised_head_shapes(fmt, hq, hkv, d):
    announce(f"{fmt} decode, Hq={hq} Hkv={hkv} d={d}")
    wl = quant_workload(fmt, hq=hq, hkv=hkv, d=d, lengths=(1, 33, 300, 700), layers=1)
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref).run()
    check(run.decode_outputs[0][0].double().cpu().numpy(), ref.attention(0, 0), f"{fmt} shape")


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
def test_quantised_qwen_layer_full(fmt):
    announce(f"{fmt}: 37 x 2304 tokens, Hq=32 Hkv=8 d=128, default launch")
    wl = replace(workloads.qwen_independent(), kv_format=fmt)
    ref = OracleReplay(wl).run()
    run = GpuRun(wl, ref=ref).run()
    check(run.decode_outputs[0][0].double().cpu().numpy(), ref.attention(0, 0), f"{fmt} 37 x 2304 layer")


def test_quantised_pool_rejects_other_kernels_and_shapes():
    announce("quantised pools: the generic kernel and B != 16 are refused")
    wl = quant_workload("q8_0", lengths=(20,), layers=1)
    run = GpuRun(wl).run()
    tables, lens = run.pool.tables([0], run.max_blocks)
    t = torch.from_numpy(tables).cuda()
    l_ = torch.from_numpy(lens).cuda()
    q = torch.zeros((1, 32, 128), dtype=torch.int16, device="cuda")
    with pytest.raises(B.KVError) as e:
        run.pool.decode(0, q, q.clone(), t, l_, 32, opts=B.attention_options(kernel=B.KV_KERNEL_GENERIC))
    assert e.value.status == B.KV_ERR_UNSUPPORTED
    with pytest.raises(B.KVError) as e:
        run.pool.prefill(0, q, q.clone(), torch.tensor([0, 1], dtype=torch.int32, device="cuda"), t, l_, 1, 32,
                         opts=B.attention_options(kernel=B.KV_KERNEL_GENERIC))
    assert e.value.status == B.KV_ERR_UNSUPPORTED
    with pytest.raises(B.KVError) as e:
        B.kv_pool_required_bytes(B.make_config(1, 4, 8, 2, 128, B.KV_Q8_0))
    assert e.value.status == B.KV_ERR_UNSUPPORTED
    torch.cuda.synchronize()
