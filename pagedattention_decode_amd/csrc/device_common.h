// Device helpers shared by the attention kernels (gfx950): bf16 conversion,
// the MFMA operand vector types and the register tile of one 16-token K/V
// block in the pool's MFMA operand order.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pagedkv {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// Round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// One 16-token block of one KV head in registers: lane l holds the 16-byte
// pieces l, l + 64, ... of the K tile and of the V tile, which are its
// operands of v_mfma_f32_16x16x32_bf16 (K as A of S^T = K Q^T) and of
// v_mfma_f32_16x16x16_bf16 (V as A of O^T = V^T P^T).
template <int D>
struct kv_regs {
  uint4 k[D / 32];
  uint4 v[D / 32];
};

template <int D>
__device__ __forceinline__ void load_block(kv_regs<D>& r, const uint4* kt, const uint4* vt, int lane) {
#pragma unroll
  for (int i = 0; i < D / 32; ++i) r.k[i] = kt[i * 64 + lane];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) r.v[i] = vt[i * 64 + lane];
}

// The running maximum m is only moved when a block's maximum exceeds it by more
// than this many binary orders of magnitude; otherwise the block is weighted
// against the stale m (weights up to 2^kRescaleSlack).  Numerator and
// denominator use the same m, so the result is unchanged; the rescale of the
// accumulators is skipped for most blocks.
constexpr float kRescaleSlack = 8.f;

// Zeroes the V values of slots >= valid of a block held in registers (their
// memory may hold anything, and a zero weight times NaN is NaN).
template <int D>
__device__ __forceinline__ void zero_v_tail(kv_regs<D>& cur, int valid, int quad) {
#pragma unroll
  for (int pp = 0; pp < D / 32; ++pp) {
    uint32_t* wv = reinterpret_cast<uint32_t*>(&cur.v[pp]);
    // 16 bytes = [half 0: 4 slots][half 1: 4 slots], 2 slots per dword
#pragma unroll
    for (int dw = 0; dw < 4; ++dw) {
      const int slot0 = quad * 4 + (dw & 1) * 2;
      uint32_t mask = 0;
      if (slot0 < valid) mask |= 0x0000ffffu;
      if (slot0 + 1 < valid) mask |= 0xffff0000u;
      wv[dw] &= mask;
    }
  }
}

}  // namespace pagedkv
