// Device helpers shared by the attention kernels (gfx950): bf16 conversion,
// the MFMA operand vector types and the register tile of one 16-token K/V
// block in the pool's MFMA operand order.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_fp16.h>
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

// Maximum and sum of x over lanes l and l ^ 16, and over l and l ^ 32, without
// the LDS pipe: v_permlane16_swap exchanges the odd 16-lane rows of its first
// operand with the even rows of its second, v_permlane32_swap the upper half
// of its first operand with the lower half of its second, so with x in both
// every lane ends up holding x[l] and its partner's value.
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// The same maxima with NaN-propagating semantics: gfx950's v_maximum3_f32
// takes its inputs as they are, where fmaxf (NaN-ignoring) first quiets every
// input that is not known to be canonical (matrix-core results, lane swaps) with
// one more instruction each.  For softmax maxima over scores, where a NaN score
// poisons its row through the weights anyway.
__device__ __forceinline__ float maxn(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float maxn3(float a, float b, float c) { return maxn(maxn(a, b), c); }
__device__ __forceinline__ float maxn_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return maxn(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float maxn_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return maxn(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// x from a partner lane by a DPP pattern within 16-lane rows: quad_perm
// [1,0,3,2] (lane ^ 1), quad_perm [2,3,0,1] (lane ^ 2), the half-row mirror
// (lane i <-> 7 - i in each 8) and the row mirror (i <-> 15 - i).
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Maximum and sum over the 64 lanes of a wave (every lane active; every lane
// gets the result): a butterfly in which every step pairs disjoint lane
// groups -- DPP within a row, then the permlane swaps across rows -- so no
// step goes through the LDS pipe.
// a / b for a >= 0, b > 0: in 32-bit arithmetic when both fit in 32 bits
// (every work-split quotient of the workloads here), which takes a small
// fraction of the instructions of the 64-bit division sequence.
__device__ __forceinline__ int64_t div_nn(int64_t a, int64_t b) {
  if (((static_cast<uint64_t>(a) | static_cast<uint64_t>(b)) >> 32) == 0)
    return static_cast<int64_t>(static_cast<uint32_t>(a) / static_cast<uint32_t>(b));
  return a / b;
}

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f32<kDppXor1>(x));
  x = fmaxf(x, dpp_f32<kDppXor2>(x));
  x = fmaxf(x, dpp_f32<kDppHalfMirror>(x));
  x = fmaxf(x, dpp_f32<kDppMirror>(x));
  return max_xor32(max_xor16(x));
}

__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f32<kDppXor1>(x);
  x += dpp_f32<kDppXor2>(x);
  x += dpp_f32<kDppHalfMirror>(x);
  x += dpp_f32<kDppMirror>(x);
  return sum_xor32(sum_xor16(x));
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

// The same for any block size: the lane's first K and V pieces at k and v, its
// i-th piece STRIDE pieces further (load_block is STRIDE = 64, k = kt + lane).
template <int D, int STRIDE>
__device__ __forceinline__ void load_block_strided(kv_regs<D>& r, const uint4* k, const uint4* v) {
#pragma unroll
  for (int i = 0; i < D / 32; ++i) r.k[i] = k[i * STRIDE];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) r.v[i] = v[i * STRIDE];
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

// ---------------------------------------------------------------------------
// Matrix-core decode step over one 16-token tile, shared by the split-K decode
// and the read-once cascade kernels.  A wave computes, for 16 query columns,
//   S^T[16 tokens][16 columns] = K[16][D] . Q^T[D][16]   (D/32 x mfma 16x16x32)
//   online softmax on S^T (each lane holds 4 tokens of one column)
//   O^T[D][16 columns] += V^T[D][16] . P^T[16][16]        (D/16 x mfma 16x16x16)
// The P^T operand is exactly the S^T result layout, so no data moves between
// lanes except the two shuffles of the per-column block maximum.
// ---------------------------------------------------------------------------

// One 16-token block: scores, online-softmax update, weighted sum of values.
// `valid` (wave uniform) is the number of in-range slots of the block.
// Online-softmax step on the 4 scores s of the lane's tokens quad*4 + i:
// masks the slots past `valid`, raises the running maximum when a score
// exceeds it by more than the slack (rescaling l and O), and returns the
// weights 2^(s * scale_log2 - m_run) (0 for masked slots).  scale_log2 > 0
// (the callers reject other scales), so the maximum of the scaled scores is
// the scaled maximum; a full block (valid = 16) needs no slot test.
template <int D>
__device__ __forceinline__ void softmax_step(const f32x4_t& s, int valid, int quad, float scale_log2, f32x4_t* o,
                                             float& m_run, float& l_lane, float (&pv)[4]) {
  float sm[4] = {s[0], s[1], s[2], s[3]};
  if (valid < 16) {  // wave uniform; the empty asm keeps this a branch, not per-slot selects
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sm[i] = quad * 4 + i < valid ? sm[i] : -INFINITY;
      asm volatile("" : "+v"(sm[i]));
    }
  }
  float mb = maxn(maxn3(sm[0], sm[1], sm[2]), sm[3]);
  mb = maxn_xor32(maxn_xor16(mb)) * scale_log2;
  const bool grow = mb > m_run + kRescaleSlack;
  if (__builtin_amdgcn_ballot_w64(grow)) {  // wave-uniform branch
    const float m_new = grow ? mb : m_run;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 when m_run = -inf, 1 when kept
    l_lane *= alpha;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) o[i] *= alpha;
    m_run = m_new;
  }
  // a masked slot (-inf) gets 2^-inf = 0; while m_run is still -inf every
  // slot of the column is masked and the offset 0 keeps that finite
  const float nm = m_run == -INFINITY ? 0.f : -m_run;
#pragma unroll
  for (int i = 0; i < 4; ++i) pv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sm[i], scale_log2, nm));
}

template <int D>
__device__ __forceinline__ void attend_block(kv_regs<D>& cur, const bf16x8_t* qop, int valid, int quad,
                                             float scale_log2, f32x4_t* o, float& m_run, float& l_lane) {
  // S^T = K . Q^T
  f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk)
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, cur.k[kk]), qop[kk], s, 0, 0, 0);

  float pv[4];
  softmax_step<D>(s, valid, quad, scale_log2, o, m_run, l_lane, pv);
  // P^T operand in bf16 (round to nearest even); the denominator sums the
  // rounded weights so that the weights applied to V are exactly normalised
  const bf16x2_t p01 = __builtin_convertvector((f32x2_t{pv[0], pv[1]}), bf16x2_t);
  const bf16x2_t p23 = __builtin_convertvector((f32x2_t{pv[2], pv[3]}), bf16x2_t);
  const uint32_t w01 = __builtin_bit_cast(uint32_t, p01);
  const uint32_t w23 = __builtin_bit_cast(uint32_t, p23);
  l_lane += (__uint_as_float(w01 << 16) + __uint_as_float(w01 & 0xffff0000u)) +
            (__uint_as_float(w23 << 16) + __uint_as_float(w23 & 0xffff0000u));
  const s16x4_t pop = __builtin_bit_cast(s16x4_t, make_uint2(w01, w23));

  // zero the values of out-of-range slots (their memory may hold anything)
  if (valid < 16) zero_v_tail<D>(cur, valid, quad);

  // O^T += V^T . P^T
#pragma unroll
  for (int pp = 0; pp < D / 32; ++pp) {
    const uint2* halves = reinterpret_cast<const uint2*>(&cur.v[pp]);
    o[2 * pp] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, halves[0]), pop, o[2 * pp],
                                                          0, 0, 0);
    o[2 * pp + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, halves[1]), pop,
                                                              o[2 * pp + 1], 0, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// Quantised tiles (B = 16, groups of 32 values along d with a half scale).
//
// One K or V tile = a code region followed by a scale region of 16 x d/32
// halves ([slot][group]).  Codes are arranged per MFMA lane: lane l = 16 q + r
// owns D*bits/32 contiguous bytes at l * D*bits/32.
//   K, lane (q, r): token r, dims 32 kk + 8 q + j (kk < D/32, j < 8);
//     q8: byte 8 kk + j; q4: byte 4 kk + j % 4, nibble j / 4 (low = j < 4).
//   V, lane (q, r): dim 16 t + r of tokens 4 q + i (t < D/16, i < 4);
//     q8: byte 4 t + i; q4: byte 4 (t/2) + i, nibble t % 2.
// A q8 code is stored as a two's-complement byte, a q4 code as code + 8.
// Every byte holds codes of one token only, so a writer owns whole bytes.
// ---------------------------------------------------------------------------

enum { kFmtBf16 = 0, kFmtQ8 = 1, kFmtQ4 = 2 };

template <int FMT>
constexpr int fmt_bits() {
  return FMT == kFmtQ8 ? 8 : 4;
}
template <int D, int FMT>
constexpr int q_code_bytes() {  // per tile
  return 16 * D * fmt_bits<FMT>() / 8;
}
template <int D, int FMT>
constexpr int q_tile_bytes() {
  return q_code_bytes<D, FMT>() + 16 * (D / 32) * 2;
}

// Raw quantised block of one KV head in registers, per lane.
template <int D, int FMT>
struct kv_qregs {
  uint32_t kc[D * fmt_bits<FMT>() / 128];  // K codes
  uint32_t vc[D * fmt_bits<FMT>() / 128];  // V codes
  uint32_t ks[D / 16];                     // K scales of the lane's 4 score tokens ([token][group])
  uint32_t vs[D / 16];                     // V scales of the same 4 tokens ([token][group])
};

template <int N>
__device__ __forceinline__ void load_dwords(uint32_t (&w)[N], const unsigned char* p) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const uint4 v = reinterpret_cast<const uint4*>(p)[i];
      w[4 * i] = v.x;
      w[4 * i + 1] = v.y;
      w[4 * i + 2] = v.z;
      w[4 * i + 3] = v.w;
    }
  } else if constexpr (N % 2 == 0) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const uint2 v = reinterpret_cast<const uint2*>(p)[i];
      w[2 * i] = v.x;
      w[2 * i + 1] = v.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) w[i] = reinterpret_cast<const uint32_t*>(p)[i];
  }
}

// Loads the lane's share of the K and V tiles at kt, vt (byte addresses).
template <int D, int FMT>
__device__ __forceinline__ void load_qblock(kv_qregs<D, FMT>& r, const unsigned char* kt, const unsigned char* vt,
                                            int lane) {
  constexpr int lane_bytes = D * fmt_bits<FMT>() / 32;
  constexpr int codes = q_code_bytes<D, FMT>();
  load_dwords(r.kc, kt + lane * lane_bytes);
  load_dwords(r.vc, vt + lane * lane_bytes);
  load_dwords(r.ks, kt + codes + (lane >> 4) * 4 * (D / 32) * 2);
  load_dwords(r.vs, vt + codes + (lane >> 4) * 4 * (D / 32) * 2);
}

__device__ __forceinline__ float half_lo(uint32_t w) { return __half2float(__ushort_as_half(static_cast<unsigned short>(w))); }
__device__ __forceinline__ float half_hi(uint32_t w) { return __half2float(__ushort_as_half(static_cast<unsigned short>(w >> 16))); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), bf16x2_t));
}

// Scale of token i (of the lane's 4) and group g, from a [token][group] list of halves.
template <int D>
__device__ __forceinline__ float scale_at(const uint32_t* w, int i, int g) {
  const int h = i * (D / 32) + g;
  return (h & 1) ? half_hi(w[h >> 1]) : half_lo(w[h >> 1]);
}

// Byte k of w as a signed integer, converted to float (one SDWA conversion).
__device__ __forceinline__ float sbyte_f32(uint32_t w, int k) {
  return static_cast<float>(static_cast<signed char>(w >> (8 * k)));
}

// q4_0 operands carry a bias: the nibble u = c + 8 becomes the bf16 value
// 128 + u = c + kQ4Bias (bit pattern 0x4300 | u, exact), so that one byte
// permute makes two operand values.  The attention step removes the bias:
// for K through the accumulator the products start from (-kQ4Bias times the
// group's query sum), for V by a second product with the constant operand
// -kQ4Bias (bf16 0xc308) on the same weights.
constexpr float kQ4Bias = 136.f;
constexpr uint32_t kQ4NegBiasPair = 0xc308c308u;

// bf16 pair (128 + b0, 128 + b1) of bytes b0 = bytes[sel], b1 = bytes[sel + 1]
// (each < 16): the permute takes 0x43 from its first operand for the high
// byte of each half.
template <int SEL>
__device__ __forceinline__ uint32_t q4_pair(uint32_t bytes) {
  constexpr uint32_t sel = 0x04000400u | static_cast<uint32_t>(SEL) | (static_cast<uint32_t>(SEL + 1) << 16);
  return __builtin_amdgcn_perm(0x43434343u, bytes, sel);
}

// The codes of a raw block as the bf16 operand tiles of the decode kernel,
// exact (integers of at most 8 significant bits).  q8_0: each two's-complement
// byte converts directly.  q4_0: the low and the high nibbles of the four
// bytes of a word, spread into bytes, give four bias pairs each (above).
// The scales themselves are applied in float32 by the attention step.
template <int D, int FMT>
__device__ __forceinline__ void codes_block(const kv_qregs<D, FMT>& r, kv_regs<D>& out) {
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    if constexpr (FMT == kFmtQ8) {
      float v[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[k] = sbyte_f32(r.kc[2 * kk], k);
        v[4 + k] = sbyte_f32(r.kc[2 * kk + 1], k);
      }
      out.k[kk] = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                             pack_bf16x2(v[6], v[7]));
    } else {
      const uint32_t lo = r.kc[kk] & 0x0f0f0f0fu;         // j = 0 .. 3
      const uint32_t hi = (r.kc[kk] >> 4) & 0x0f0f0f0fu;  // j = 4 .. 7
      out.k[kk] = make_uint4(q4_pair<0>(lo), q4_pair<2>(lo), q4_pair<0>(hi), q4_pair<2>(hi));
    }
  }
  // V: tile t gives the 16x16x16 operand of dims 16 t + r for the lane's 4 tokens
  uint32_t half_words[D / 16][2];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    if constexpr (FMT == kFmtQ8) {
      const uint32_t bytes = r.vc[t];
      half_words[t][0] = pack_bf16x2(sbyte_f32(bytes, 0), sbyte_f32(bytes, 1));
      half_words[t][1] = pack_bf16x2(sbyte_f32(bytes, 2), sbyte_f32(bytes, 3));
    } else {
      const uint32_t bytes = (t & 1) ? ((r.vc[t >> 1] >> 4) & 0x0f0f0f0fu) : (r.vc[t >> 1] & 0x0f0f0f0fu);
      half_words[t][0] = q4_pair<0>(bytes);
      half_words[t][1] = q4_pair<2>(bytes);
    }
  }
#pragma unroll
  for (int pp = 0; pp < D / 32; ++pp)
    out.v[pp] = make_uint4(half_words[2 * pp][0], half_words[2 * pp][1], half_words[2 * pp + 1][0],
                           half_words[2 * pp + 1][1]);
}

// Launches a kernel; with a start or stop event, through hipExtLaunchKernel so
// that the events take the kernel's own timestamps.
template <typename F, typename... Args>
hipError_t launch_timed(F kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t st, hipEvent_t ev_start,
                        hipEvent_t ev_stop, Args... args) {
  if (ev_start || ev_stop) {
    hipExtLaunchKernelGGL(kernel, grid, block, lds, st, ev_start, ev_stop, 0u, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, lds, st, args...);
  }
  return hipGetLastError();
}

}  // namespace pagedkv
