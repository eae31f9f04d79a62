"""Grouped 8- and 4-bit KV quantisation (test infrastructure; see oracle/__init__).

[INF] section 8.4.2 and Figure 8-23: 32 BF16 values take 64 bytes; q8_0 keeps
32 one-byte codes and one 2-byte scale per group of 32 values (34 bytes,
8.5 bits per value), q4_0 the same grouping with 4-bit codes (16 + 2 = 18
bytes, 4.5 bits per value); a context's KV footprint scales by 34/64 and
18/64.  Reading a compressed KV saves Delta D bytes at effective bandwidth
beta and costs a conversion time T_c: the net saving is Delta D / beta - T_c.

The pages give the byte budget, not the arithmetic of the codes.  Readings
taken here (the plainest that fits that budget):

* a group is 32 consecutive values along the head dimension of one token of
  one KV head (values are produced and written token by token);
* symmetric absmax scaling: scale = max|x| / 127 (q8_0) or / 7 (q4_0),
  computed in float32 and stored as IEEE half (the 2-byte scale), saturated to
  the largest finite half; codes = x / scale_half in float32, rounded to
  nearest with ties to even, clamped to [-127, 127] or [-7, 7]; a group whose
  scale is 0 has all codes 0;
* q4_0 stores code + 8 in a nibble, the even value of a pair in the low
  nibble;
* a value is read back as code * scale.

Floating point decides the integer codes, so this module takes those steps
in float32 exactly as written, like the kernel that writes the pool.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

GROUP = 32
FORMATS = {"q8_0": (8, 127), "q4_0": (4, 7)}  # code bits, largest code magnitude
HALF_MAX = 65504.0


def group_bytes(fmt: str) -> int:
    """Bytes of one group of 32 values: codes plus a 2-byte scale ([INF] Figure 8-23)."""
    bits, _ = FORMATS[fmt]
    return GROUP * bits // 8 + 2


def bits_per_value(fmt: str) -> Fraction:
    return Fraction(8 * group_bytes(fmt), GROUP)


def footprint_ratio(fmt: str) -> Fraction:
    """Quantised bytes over BF16 bytes for the same values (64 bytes per group in BF16)."""
    return Fraction(group_bytes(fmt), 2 * GROUP)


def quantized_bytes(bf16_bytes, fmt: str) -> Fraction:
    return Fraction(bf16_bytes) * footprint_ratio(fmt)


def net_saving(saved_bytes, bandwidth, conversion_time):
    """Delta T = Delta D / beta - T_c ([INF] section 8.4.2)."""
    return saved_bytes / bandwidth - conversion_time


def linear_crossover(fixed_a, per_token_a, fixed_b, per_token_b):
    """Context length where two fits t = fixed + per_token * L meet."""
    return (fixed_b - fixed_a) / (per_token_a - per_token_b)


def quantize(x, fmt: str):
    """x: float values [..., n] with n a multiple of 32 (exact in float32).

    Returns (codes int8 [..., n], scales uint16 half bits [..., n / 32]).
    """
    _, qmax = FORMATS[fmt]
    x = np.asarray(x, dtype=np.float32)
    if x.shape[-1] % GROUP:
        raise ValueError("the last dimension must be a multiple of 32")
    g = x.reshape(x.shape[:-1] + (x.shape[-1] // GROUP, GROUP))
    amax = np.abs(g).max(axis=-1)
    s32 = amax / np.float32(qmax)                       # float32 division
    s32 = np.minimum(s32, np.float32(HALF_MAX))
    s16 = s32.astype(np.float16)                        # round to nearest even, subnormals kept
    sf = s16.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = g / sf[..., None]                       # float32 division
    codes = np.where(sf[..., None] > 0, np.rint(ratio), 0.0)
    codes = np.clip(codes, -qmax, qmax).astype(np.int8)
    return codes.reshape(x.shape), s16.view(np.uint16)


def dequantize(codes, scales):
    """code * scale, exactly, in float64 ([..., n], [..., n / 32] half bits)."""
    codes = np.asarray(codes, dtype=np.float64)
    s = np.asarray(scales, dtype=np.uint16).view(np.float16).astype(np.float64)
    g = codes.reshape(codes.shape[:-1] + (codes.shape[-1] // GROUP, GROUP))
    return (g * s[..., None]).reshape(codes.shape)


def pack_q4(codes):
    """int8 codes in [-7, 7], even count along the last axis -> bytes (code + 8, low nibble first)."""
    c = (np.asarray(codes, dtype=np.int16) + 8).astype(np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_q4(packed):
    p = np.asarray(packed, dtype=np.uint8)
    lo = (p & 0x0F).astype(np.int16) - 8
    hi = (p >> 4).astype(np.int16) - 8
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


class QuantKVStore:
    """Logical pool of a quantised cache (same interface as :class:`oracle.kv_store.KVStore`).

    Per (layer, block): codes int8 [B, Hkv, d] and scales as half bits
    [B, Hkv, d / 32]; a token row is quantised group by group when written.
    Rows arrive as the stored bit patterns of their source dtype (``src_dtype``)
    and are widened exactly before quantisation.  Unwritten blocks hold codes 0
    and scales 0.
    """

    def __init__(self, num_layers, num_blocks, block_size, num_kv_heads, head_dim, fmt, src_dtype, layers=None):
        from synth import draws  # widening of stored bit patterns only

        self._widen = lambda bits: draws.bits_to_f64(bits, src_dtype).astype(np.float32)
        self.fmt = fmt
        self.num_layers = num_layers
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.num_kv_heads = num_kv_heads
        self.head_dim = head_dim
        self.layers = None if layers is None else set(layers)
        self.k: dict = {}
        self.v: dict = {}

    def _tracked(self, layer) -> bool:
        return self.layers is None or layer in self.layers

    def _empty(self):
        B, H, d = self.block_size, self.num_kv_heads, self.head_dim
        return (np.zeros((B, H, d), np.int8), np.zeros((B, H, d // GROUP), np.uint16))

    def _block(self, store, layer, block, create):
        key = (layer, block)
        blk = store.get(key)
        if blk is None:
            blk = self._empty()
            if create:
                store[key] = blk
        return blk

    def write(self, layer, slots, k_rows, v_rows) -> None:
        if not self._tracked(layer):
            return
        kc, ks = quantize(self._widen(k_rows), self.fmt)
        vc, vs = quantize(self._widen(v_rows), self.fmt)
        for i, slot in enumerate(slots):
            if slot < 0:
                continue
            block, offset = divmod(int(slot), self.block_size)
            codes, scales = self._block(self.k, layer, block, True)
            codes[offset], scales[offset] = kc[i], ks[i]
            codes, scales = self._block(self.v, layer, block, True)
            codes[offset], scales[offset] = vc[i], vs[i]

    def copy_blocks(self, pairs) -> None:
        for layer in range(self.num_layers):
            if not self._tracked(layer):
                continue
            for src, dst in pairs:
                for store in (self.k, self.v):
                    c, s = self._block(store, layer, src, False)
                    store[(layer, dst)] = (c.copy(), s.copy())

    def block(self, which, layer, block):
        """(codes [B, Hkv, d] int8, scales [B, Hkv, d / 32] half bits) of one block."""
        return self._block(self.k if which == "k" else self.v, layer, block, False)

    def to_host(self, pairs) -> None:
        """(block, frame) pairs: frame := block (codes and scales), every tracked layer."""
        if not hasattr(self, "host_k"):
            self.host_k, self.host_v = {}, {}
        for layer in range(self.num_layers):
            if not self._tracked(layer):
                continue
            for block, frame in pairs:
                for store, host in ((self.k, self.host_k), (self.v, self.host_v)):
                    c, s = self._block(store, layer, block, False)
                    host[(layer, frame)] = (c.copy(), s.copy())

    def from_host(self, pairs) -> None:
        """(frame, block) pairs: block := frame, every tracked layer."""
        for layer in range(self.num_layers):
            if not self._tracked(layer):
                continue
            for frame, block in pairs:
                for store, host in ((self.k, self.host_k), (self.v, self.host_v)):
                    c, s = host[(layer, frame)]
                    store[(layer, block)] = (c.copy(), s.copy())

    def host_block(self, which, layer, frame):
        return (self.host_k if which == "k" else self.host_v)[(layer, frame)]

    def gather_f64(self, layer, table, n):
        """Dequantised K and V rows [n, Hkv, d] float64 of a sequence of length n."""
        k = np.empty((n, self.num_kv_heads, self.head_dim))
        v = np.empty_like(k)
        for t in range(0, n, self.block_size):
            j = t // self.block_size
            take = min(self.block_size, n - t)
            kc, ksc = self.block("k", layer, table[j])
            vc, vsc = self.block("v", layer, table[j])
            k[t:t + take] = dequantize(kc[:take], ksc[:take])
            v[t:t + take] = dequantize(vc[:take], vsc[:take])
        return k, v
