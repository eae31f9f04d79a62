// Device side of the paged KV cache for gfx950 (MI355X): slot scatter, block
// copy, decode attention over block tables (split-K partitions) and the
// log-sum-exp merge.
//
// Sources (by page title):
//   [BT]  "PagedAttention 的块表与碎片控制": §03 j = t / B, r = t mod B,
//         p = block_table[j]; §06 caches [layers, blocks, B, Hkv, d] as the
//         readable form (the stride is left to the kernel); §07 decode
//         equation s_t = q . k_t / sqrt(d), o = sum softmax(s)_t v_t, combined
//         blockwise with an online softmax.
//   [KVM] "KV 缓存管理": paged KV allocation (K/V of a new token written to
//         T[l] at offset o; the decode kernel takes the block table as an extra
//         input and walks logical blocks 0 .. floor((S-1)/B)); copy-on-write
//         (copy the B tokens of the shared block); chunked prefill mechanism
//         (running max m, sum l and output O folded across blocks).
//
// Pool layout: see include/pagedkv.h.  Per (layer, block, kv head) one tile of
// B*d elements; K tile = [d/X][B][X] (X = 16 bytes of elements), V tile =
// [d/32][B/Q][16][2][Q] (Q = gcd(B, 4)).  For bf16, B = 16 these are exactly the
// register operand orders of v_mfma_f32_16x16x32_bf16 (K, as the A operand of
// S^T = K Q^T) and v_mfma_f32_16x16x16_bf16 (V, as the A operand of
// O^T = V^T P^T), so every K/V byte is fetched by one 16-byte load per lane and
// every wave-wide load instruction reads 1 KiB of contiguous memory.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <string>
#include <type_traits>

#include "device_common.h"
#include "pool_internal.h"

namespace pagedkv {
namespace {

// ---------------------------------------------------------------------------
// element helpers
// ---------------------------------------------------------------------------

template <typename T> struct elem;
template <> struct elem<float> {
  __device__ static float to_f32(float x) { return x; }
  __device__ static float from_f32(float x) { return x; }
};
template <> struct elem<uint16_t> {
  __device__ static float to_f32(uint16_t x) { return bf16_to_f32(x); }
  __device__ static uint16_t from_f32(float x) { return f32_to_bf16(x); }
};

// Element offset of (slot r, dim e) inside a K tile.
__device__ __forceinline__ int k_offset(int r, int e, int B, int X) { return ((e / X) * B + r) * X + (e % X); }

// Element offset of (slot r, dim e) inside a V tile.
__device__ __forceinline__ int v_offset(int r, int e, int B, int Q) {
  return ((((e >> 5) * (B / Q) + r / Q) * 16 + (e & 15)) * 2 + ((e & 31) >> 4)) * Q + r % Q;
}

// ---------------------------------------------------------------------------
// reshape_and_cache: one thread per 16-byte chunk of a new K row; the same
// thread scatters the matching V elements.
// ---------------------------------------------------------------------------

template <typename T>
__global__ void __launch_bounds__(256) reshape_and_cache_kernel(
    const T* __restrict__ k_new, const T* __restrict__ v_new, const int64_t* __restrict__ slots,
    T* __restrict__ k_layer, T* __restrict__ v_layer, int64_t n_items, int n_kv_heads, int head_dim,
    int block_size, int64_t n_slots) {
  constexpr int X = 16 / sizeof(T);
  const int Q = (block_size % 4 == 0) ? 4 : ((block_size % 2 == 0) ? 2 : 1);
  const int chunks_per_head = head_dim / X;
  const int64_t chunks_per_token = static_cast<int64_t>(n_kv_heads) * chunks_per_head;
  for (int64_t item = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; item < n_items;
       item += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t tok = item / chunks_per_token;
    const int rem = static_cast<int>(item % chunks_per_token);
    const int g = rem / chunks_per_head;
    const int c = rem % chunks_per_head;
    // the new rows are read together with the slot (they are in bounds whatever the slot is),
    // so the two loads wait out one memory latency, not two
    const int64_t src = (tok * n_kv_heads + g) * head_dim + static_cast<int64_t>(c) * X;
    const uint4 kv = *reinterpret_cast<const uint4*>(k_new + src);
    const uint4 vv = *reinterpret_cast<const uint4*>(v_new + src);
    const int64_t slot = slots[tok];
    if (slot < 0 || slot >= n_slots) continue;
    const int64_t blk = slot / block_size;
    const int r = static_cast<int>(slot % block_size);
    const int64_t tile = (blk * n_kv_heads + g) * static_cast<int64_t>(block_size) * head_dim;
    // K: one 16-byte chunk, contiguous in the tile
    *reinterpret_cast<uint4*>(k_layer + tile + k_offset(r, c * X, block_size, X)) = kv;
    // V: X elements, each to its own place
    const T* ve = reinterpret_cast<const T*>(&vv);
#pragma unroll
    for (int x = 0; x < X; ++x) v_layer[tile + v_offset(r, c * X + x, block_size, Q)] = ve[x];
  }
}

// ---------------------------------------------------------------------------
// reshape_and_cache into a quantised pool ([INF] §8.4.2: 32 values share one
// 2-byte scale): one thread per (token, KV head, group of 32 dims).  It forms
// the group's half scale max|x| / M and codes rint(x / s) for K and for V and
// writes them in the tile layout of device_common.h; every byte it writes
// holds codes of its own token only.
// ---------------------------------------------------------------------------

template <int D, int FMT>
__device__ __forceinline__ void quantize_group(const uint16_t* __restrict__ x, float* c, uint16_t& scale_bits) {
  constexpr float qmax = FMT == kFmtQ8 ? 127.f : 7.f;
  float f[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 w = reinterpret_cast<const uint4*>(x)[i];
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      f[8 * i + 2 * k] = __uint_as_float(ws[k] << 16);
      f[8 * i + 2 * k + 1] = __uint_as_float(ws[k] & 0xffff0000u);
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(f[i]));
  const __half hs = __float2half_rn(fminf(__fdiv_rn(amax, qmax), 65504.f));
  scale_bits = __half_as_ushort(hs);
  const float s = __half2float(hs);
#pragma unroll
  for (int i = 0; i < 32; ++i) c[i] = s > 0.f ? fminf(fmaxf(rintf(__fdiv_rn(f[i], s)), -qmax), qmax) : 0.f;
}

template <int D, int FMT>
__global__ void __launch_bounds__(256) quantize_cache_kernel(const uint16_t* __restrict__ k_new,
                                                             const uint16_t* __restrict__ v_new,
                                                             const int64_t* __restrict__ slots,
                                                             unsigned char* __restrict__ k_layer,
                                                             unsigned char* __restrict__ v_layer, int64_t n_items,
                                                             int n_kv_heads, int64_t n_slots) {
  constexpr int G32 = D / 32;
  constexpr int TB = q_tile_bytes<D, FMT>();
  constexpr int CB = q_code_bytes<D, FMT>();
  constexpr int LB = D * fmt_bits<FMT>() / 32;  // code bytes per lane
  for (int64_t item = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; item < n_items;
       item += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t tok = item / (n_kv_heads * G32);
    const int rem = static_cast<int>(item % (n_kv_heads * G32));
    const int h = rem / G32, grp = rem % G32;
    const int64_t slot = slots[tok];
    if (slot < 0 || slot >= n_slots) continue;
    const int r = static_cast<int>(slot & 15);
    const int64_t tile = ((slot >> 4) * n_kv_heads + h) * TB;
    const int64_t src = (tok * n_kv_heads + h) * D + grp * 32;
    float c[32];
    uint16_t sb;
    // K: lane (q, r) holds dims 32 grp + 8 q + j
    quantize_group<D, FMT>(k_new + src, c, sb);
    unsigned char* kt = k_layer + tile;
    *reinterpret_cast<uint16_t*>(kt + CB + (r * G32 + grp) * 2) = sb;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      unsigned char* dst = kt + (q * 16 + r) * LB;
      if constexpr (FMT == kFmtQ8) {
        uint32_t w[2] = {0u, 0u};
#pragma unroll
        for (int j = 0; j < 8; ++j) w[j >> 2] |= (static_cast<uint32_t>(static_cast<int>(c[q * 8 + j])) & 0xffu) << (8 * (j & 3));
        *reinterpret_cast<uint2*>(dst + grp * 8) = make_uint2(w[0], w[1]);
      } else {
        uint32_t w = 0u;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          w |= static_cast<uint32_t>(static_cast<int>(c[q * 8 + j]) + 8) << (8 * (j % 4) + 4 * (j / 4));
        *reinterpret_cast<uint32_t*>(dst + grp * 4) = w;
      }
    }
    // V: lane (r / 4, rr) holds dim 16 t + rr of this token (slot r % 4 of its four)
    quantize_group<D, FMT>(v_new + src, c, sb);
    unsigned char* vt = v_layer + tile;
    *reinterpret_cast<uint16_t*>(vt + CB + (r * G32 + grp) * 2) = sb;
    const int qv = r >> 2, i = r & 3;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      unsigned char* dst = vt + (qv * 16 + rr) * LB;
      if constexpr (FMT == kFmtQ8) {
        dst[(2 * grp) * 4 + i] = static_cast<unsigned char>(static_cast<int>(c[rr]));
        dst[(2 * grp + 1) * 4 + i] = static_cast<unsigned char>(static_cast<int>(c[16 + rr]));
      } else {
        dst[grp * 4 + i] = static_cast<unsigned char>((static_cast<int>(c[rr]) + 8) |
                                                      ((static_cast<int>(c[16 + rr]) + 8) << 4));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// copy_blocks: one workgroup per (pair, layer, K or V); copies the Hkv tiles of
// that block, which are contiguous.
// ---------------------------------------------------------------------------

__global__ void __launch_bounds__(256) copy_blocks_kernel(uint4* __restrict__ k_pool, uint4* __restrict__ v_pool,
                                                          const int64_t* __restrict__ pairs, int num_layers,
                                                          int num_blocks, int64_t block_vec16) {
  const int pair = blockIdx.x / (num_layers * 2);
  const int rem = blockIdx.x % (num_layers * 2);
  const int layer = rem >> 1;
  uint4* base = (rem & 1) ? v_pool : k_pool;
  const int64_t src = pairs[2 * pair];
  const int64_t dst = pairs[2 * pair + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const uint4* s = base + (static_cast<int64_t>(layer) * num_blocks + src) * block_vec16;
  uint4* d = base + (static_cast<int64_t>(layer) * num_blocks + dst) * block_vec16;
  for (int64_t i = threadIdx.x; i < block_vec16; i += blockDim.x) d[i] = s[i];
}

// ---------------------------------------------------------------------------
// Shared by both attention kernels: the work item of a workgroup and the
// per-partition output (final row when the sequence has one partition, else
// the partial (m, l, o) of the running-max recurrences, with m in base-2
// units because scores are pre-multiplied by log2(e)).
// ---------------------------------------------------------------------------

struct attn_args {
  const void* q;
  void* out;
  const int32_t* tables;
  const int32_t* ctx_lens;
  const void* k_layer;
  const void* v_layer;
  float* part_m;  // [n_seqs][Hq][max_parts]
  float* part_l;  // [n_seqs][Hq][max_parts]
  float* part_o;  // [n_seqs][Hq][max_parts][d]
  int n_seqs, max_blocks, n_q_heads, n_kv_heads, head_dim, block_size, num_blocks;
  int partition_tokens, max_parts;
  float scale_log2;  // scale * log2(e)
  // row of `tables` that sequence s reads (NULL: row s); a negative row has
  // no valid entry (the sequence's output is NaN)
  const int32_t* table_rows;
};

struct work_item {
  int seq, kv_head, part, n, n_parts, tok_begin, tok_end;
};

__device__ __forceinline__ bool decode_work(const attn_args& a, work_item& w) {
  // Workgroups are numbered (part, kv head, seq) with seq fastest, so the
  // workgroups running together read the same partition index of different
  // sequences (sequences sharing a prefix then read the same blocks together).
  int id = blockIdx.x;
  w.seq = id % a.n_seqs;
  id /= a.n_seqs;
  w.kv_head = id % a.n_kv_heads;
  w.part = id / a.n_kv_heads;
  int n = a.ctx_lens[w.seq];
  const int cap = a.max_blocks * a.block_size;
  w.n = n > cap ? cap : n;
  w.n_parts = w.n <= 0 ? 1 : (w.n + a.partition_tokens - 1) / a.partition_tokens;
  if (w.part >= w.n_parts) return false;
  w.tok_begin = w.part * a.partition_tokens;
  w.tok_end = min(w.n, w.tok_begin + a.partition_tokens);
  return true;
}

template <typename T>
__device__ __forceinline__ void store_result(const attn_args& a, const work_item& w, int h_local, int e, float m,
                                             float l, float o, bool poisoned) {
  const int G = a.n_q_heads / a.n_kv_heads;
  const int h = w.kv_head * G + h_local;
  if (w.n_parts == 1) {
    float val = (w.n <= 0) ? 0.f : o / l;
    if (poisoned) val = __builtin_nanf("");
    T* out = static_cast<T*>(a.out);
    out[(static_cast<int64_t>(w.seq) * a.n_q_heads + h) * a.head_dim + e] = elem<T>::from_f32(val);
  } else {
    const int64_t ph = (static_cast<int64_t>(w.seq) * a.n_q_heads + h) * a.max_parts + w.part;
    if (poisoned) {
      m = l = o = __builtin_nanf("");
    }
    if (e == 0) {
      a.part_m[ph] = m;
      a.part_l[ph] = l;
    }
    a.part_o[ph * a.head_dim + e] = o;
  }
}

// ---------------------------------------------------------------------------
// Generic decode attention (vector ALU).  Any dtype, block size, head_dim
// (multiple of 32, <= 256) and group G <= 16.  A workgroup of 4 waves handles
// one (sequence, kv head, partition); each wave takes 64 tokens at a time, one
// token per lane for the scores (q in LDS), then one dimension per lane for
// the weighted sum of values.
// ---------------------------------------------------------------------------

constexpr int kGenericWaves = 4;

template <typename T, int D>
__global__ void __launch_bounds__(256) attn_generic_kernel(attn_args a) {
  constexpr int X = 16 / sizeof(T);
  constexpr int DPL = (D + 63) / 64;  // dims per lane in the PV phase
  __shared__ float q_s[kMaxGroup][D];  // scaled queries; reused for the merged output
  __shared__ float p_s[kGenericWaves][kMaxGroup][64];
  __shared__ int64_t base_s[kGenericWaves][64];
  __shared__ int r_s[kGenericWaves][64];
  __shared__ float m_s[kGenericWaves][kMaxGroup], l_s[kGenericWaves][kMaxGroup];
  __shared__ int poison_s;

  work_item w;
  if (!decode_work(a, w)) return;
  const int G = a.n_q_heads / a.n_kv_heads;
  const int B = a.block_size;
  const int Q = (B % 4 == 0) ? 4 : ((B % 2 == 0) ? 2 : 1);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const T* qg = static_cast<const T*>(a.q) + (static_cast<int64_t>(w.seq) * a.n_q_heads + w.kv_head * G) * D;
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) q_s[i / D][i % D] = elem<T>::to_f32(qg[i]) * a.scale_log2;
  if (threadIdx.x == 0) poison_s = 0;
  __syncthreads();

  const T* kl = static_cast<const T*>(a.k_layer);
  const T* vl = static_cast<const T*>(a.v_layer);
  const int trow = a.table_rows ? a.table_rows[w.seq] : w.seq;
  const int32_t* table = a.tables + static_cast<int64_t>(max(trow, 0)) * a.max_blocks;
  const int64_t tile_elems = static_cast<int64_t>(B) * D;

  float m_run[kMaxGroup], l_lane[kMaxGroup], acc[kMaxGroup][DPL];
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    m_run[h] = -INFINITY;
    l_lane[h] = 0.f;
#pragma unroll
    for (int k = 0; k < DPL; ++k) acc[h][k] = 0.f;
  }
  bool poisoned = false;

  const int span = w.tok_end - w.tok_begin;
  const int rounds = (span + 64 * kGenericWaves - 1) / (64 * kGenericWaves);
  for (int rd = 0; rd < rounds; ++rd) {
    const int t0 = w.tok_begin + (rd * kGenericWaves + wave) * 64;
    const int t = t0 + lane;
    bool valid = t < w.tok_end;
    int64_t base = 0;
    int r = 0;
    if (valid) {
      const int p = trow >= 0 ? table[t / B] : -1;
      r = t % B;
      if (p < 0 || p >= a.num_blocks) {
        valid = false;
        poisoned = true;
      } else {
        base = (static_cast<int64_t>(p) * a.n_kv_heads + w.kv_head) * tile_elems;
      }
    }
    float s[kMaxGroup];
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) s[h] = 0.f;
    if (valid) {
      for (int c = 0; c < D / X; ++c) {
        const uint4 raw = *reinterpret_cast<const uint4*>(kl + base + k_offset(r, c * X, B, X));
        const T* ke = reinterpret_cast<const T*>(&raw);
#pragma unroll
        for (int x = 0; x < X; ++x) {
          const float kx = elem<T>::to_f32(ke[x]);
#pragma unroll
          for (int h = 0; h < kMaxGroup; ++h)
            if (h < G) s[h] += q_s[h][c * X + x] * kx;
        }
      }
    }
    base_s[wave][lane] = base;
    r_s[wave][lane] = valid ? r : -1;
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
      if (h >= G) continue;
      const float sv = valid ? s[h] : -INFINITY;
      const float mc = wave_max(sv);
      const float m_new = fmaxf(m_run[h], mc);
      float alpha = 1.f, pv = 0.f;
      if (m_new != -INFINITY) {
        alpha = exp2f(m_run[h] - m_new);
        pv = valid ? exp2f(sv - m_new) : 0.f;
      }
      m_run[h] = m_new;
      l_lane[h] = l_lane[h] * alpha + pv;
      p_s[wave][h][lane] = pv;
#pragma unroll
      for (int k = 0; k < DPL; ++k) acc[h][k] *= alpha;
    }
    __syncthreads();
    const int nvalid = min(64, max(0, w.tok_end - t0));
    for (int i = 0; i < nvalid; ++i) {
      const int ri = r_s[wave][i];
      if (ri < 0) continue;
      const int64_t bi = base_s[wave][i];
#pragma unroll
      for (int k = 0; k < DPL; ++k) {
        const int e = lane + 64 * k;
        if (e < D) {
          const float vx = elem<T>::to_f32(vl[bi + v_offset(ri, e, B, Q)]);
#pragma unroll
          for (int h = 0; h < kMaxGroup; ++h)
            if (h < G) acc[h][k] += p_s[wave][h][i] * vx;
        }
      }
    }
    __syncthreads();
  }

  // merge the waves of the workgroup: common maximum per head, then the waves
  // add their rescaled partial outputs into q_s (no longer needed) in a fixed
  // order, one wave at a time, so the result is the same bits on every run
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    if (h >= G) continue;
    const float lw = wave_sum(l_lane[h]);
    if (lane == 0) {
      m_s[wave][h] = m_run[h];
      l_s[wave][h] = lw;
    }
  }
  if (poisoned) atomicOr(&poison_s, 1);
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) q_s[i / D][i % D] = 0.f;
  __syncthreads();
  for (int turn = 0; turn < kGenericWaves; ++turn) {
    if (wave == turn) {
#pragma unroll
      for (int h = 0; h < kMaxGroup; ++h) {
        if (h >= G) continue;
        float M = -INFINITY;
        for (int v = 0; v < kGenericWaves; ++v) M = fmaxf(M, m_s[v][h]);
        const float f = (M == -INFINITY) ? 0.f : exp2f(m_run[h] - M);
#pragma unroll
        for (int k = 0; k < DPL; ++k) {
          const int e = lane + 64 * k;
          if (e < D) q_s[h][e] += acc[h][k] * f;
        }
      }
    }
    __syncthreads();
  }
  const bool any_poison = poison_s != 0;
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
    const int h = i / D, e = i % D;
    float M = -INFINITY;
    for (int v = 0; v < kGenericWaves; ++v) M = fmaxf(M, m_s[v][h]);
    float L = 0.f;
    if (M != -INFINITY)
      for (int v = 0; v < kGenericWaves; ++v) L += exp2f(m_s[v][h] - M) * l_s[v][h];
    store_result<T>(a, w, h, e, M, L, q_s[h][e], any_poison);
  }
}

// ---------------------------------------------------------------------------
// Matrix-core decode attention: bf16 (any B of 4 .. 64) or quantised (B = 16),
// d = D, G <= 16 query heads as the 16 columns of one tile; heads beyond G are
// zero columns whose results are discarded.  The per-tile step (attend_block)
// is in device_common.h; the quantised variant follows.
// ---------------------------------------------------------------------------


// The same step on a quantised block, with the codes (exact in bf16) as the
// operands and the group scales applied in float32:
//   score(r) = sum_g sK(r, g) * (codes_K(r, group g) . q(group g)),
//   O      += sum_r  p(r) * sV(r, g) * codes_V(r, dims of group g),
// so the only rounding beyond float32 is that of the weight p * sV to bf16
// (the unquantised path rounds p alone).  l sums the unrounded weights.
// q4_0 tiles hold code + kQ4Bias: kbias[kk] (-kQ4Bias times the sum of the
// query over group kk, per column) starts each score product, and every V
// product is followed by one with the constant -kQ4Bias on the same weights,
// so both cancel within the tile (products of bf16 values are exact, the
// accumulation is float32).  q8_0 passes zeros.
template <int D, int FMT>
__device__ __forceinline__ void attend_qblock(const kv_regs<D>& cur, const kv_qregs<D, FMT>& raw,
                                              const bf16x8_t* qop, const f32x4_t* kbias, int valid, int quad,
                                              float scale_log2, f32x4_t* o, float& m_run, float& l_lane) {
  // each product is one mixed-precision fma on the half scale
  f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {  // one group of 32 dims per instruction
    const f32x4_t t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, cur.k[kk]), qop[kk],
                                                               kbias[kk], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = __builtin_fmaf(scale_at<D>(raw.ks, i, kk), t[i], s[i]);
  }
  float pv[4];
  softmax_step<D>(s, valid, quad, scale_log2, o, m_run, l_lane, pv);
  l_lane += (pv[0] + pv[1]) + (pv[2] + pv[3]);
  // O^T += V^T . (P * sV)^T, one weight operand per group.  The weight is one
  // mixed-precision fma p * sV + 0; a masked slot (only in a partial tile)
  // gets weight 0 by selection, as its scale and codes may be anything
#pragma unroll
  for (int pp = 0; pp < D / 32; ++pp) {
    float w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = __builtin_fmaf(scale_at<D>(raw.vs, i, pp), pv[i], 0.f);
    if (valid < 16) {  // wave uniform
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = pv[i] == 0.f ? 0.f : w[i];
    }
    const s16x4_t pop = __builtin_bit_cast(s16x4_t, make_uint2(pack_bf16x2(w[0], w[1]), pack_bf16x2(w[2], w[3])));
    const uint2* halves = reinterpret_cast<const uint2*>(&cur.v[pp]);
    o[2 * pp] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, halves[0]), pop, o[2 * pp],
                                                          0, 0, 0);
    o[2 * pp + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, halves[1]), pop,
                                                              o[2 * pp + 1], 0, 0, 0);
    if constexpr (FMT == kFmtQ4) {
      const s16x4_t nb = __builtin_bit_cast(s16x4_t, make_uint2(kQ4NegBiasPair, kQ4NegBiasPair));
      o[2 * pp] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(nb, pop, o[2 * pp], 0, 0, 0);
      o[2 * pp + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(nb, pop, o[2 * pp + 1], 0, 0, 0);
    }
  }
}

// ---------------------------------------------------------------------------
// The same decode step with vector-ALU dot products instead of matrix
// instructions (bf16, B = 16, GT query heads per KV head, compile time), on
// the tile exactly as the ring loads it: lane (r, q) = (lane % 16, lane / 16)
// holds D/4 dims of key r (k[kk]: dims 32 kk + 8 q .. + 8) and, for every
// 16-dim tile t, the values of tokens 4q .. 4q+3 in dim 16 t + r (v[t / 2],
// 8-byte half t % 2).
//   scores   s(r, h): 4 v_dot2_f32_bf16 per 8 dims against the unit's queries
//            (LDS, broadcast reads), then summed over the four quads by the
//            two lane swaps, so every quad holds the scores of key r;
//   softmax  the block maximum per head over the 16 keys of a row (DPP within
//            the row), the same lazy rescale and bf16 weights as the matrix
//            path; the weights of keys (r, r + 1) are packed in lane r;
//   values   lane (r, q) fetches the packed weights of its tokens 4q .. 4q+3
//            (two ds_bpermute per head) and adds them into acc[h][t] with two
//            v_dot2_f32_bf16 per head and tile.
// acc[h][t] sums over the lane's token slots only; the four quads' sums are
// added when the unit's run ends.  l[h] sums, per lane, the weights of key r
// (the quads hold copies; a row's 16 lanes are added at the end).
// ---------------------------------------------------------------------------
template <int D, int GT>
struct valu_state {
  float acc[GT][D / 16];
  float m[GT];
  float l[GT];
};

template <int D, int GT>
__device__ __forceinline__ void valu_reset(valu_state<D, GT>& st) {
#pragma unroll
  for (int h = 0; h < GT; ++h) {
#pragma unroll
    for (int t = 0; t < D / 16; ++t) st.acc[h][t] = 0.f;
    st.m[h] = -INFINITY;
    st.l[h] = 0.f;
  }
}

// maximum over the 16 lanes of each row (every lane gets its row's)
__device__ __forceinline__ float row_max16(float x) {
  x = maxn(x, dpp_f32<kDppXor1>(x));
  x = maxn(x, dpp_f32<kDppXor2>(x));
  x = maxn(x, dpp_f32<kDppHalfMirror>(x));
  return maxn(x, dpp_f32<kDppMirror>(x));
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_f32<kDppXor1>(x);
  x += dpp_f32<kDppXor2>(x);
  x += dpp_f32<kDppHalfMirror>(x);
  return x + dpp_f32<kDppMirror>(x);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

template <int D, int GT>
__device__ __forceinline__ void attend_block_valu(kv_regs<D>& cur, const uint16_t* qs, int valid, int lane,
                                                  float scale_log2, valu_state<D, GT>& st) {
  const int r = lane & 15, q = lane >> 4;
  // the values of out-of-range slots are zeroed (their memory may hold anything)
  if (valid < 16) zero_v_tail<D>(cur, valid, q);
  float s[GT];
#pragma unroll
  for (int h = 0; h < GT; ++h) s[h] = 0.f;
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    const uint4 k4 = cur.k[kk];
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      const uint4 q4 = *reinterpret_cast<const uint4*>(qs + h * D + kk * 32 + q * 8);
      s[h] = dot2_bf16(k4.x, q4.x, s[h]);
      s[h] = dot2_bf16(k4.y, q4.y, s[h]);
      s[h] = dot2_bf16(k4.z, q4.z, s[h]);
      s[h] = dot2_bf16(k4.w, q4.w, s[h]);
    }
  }
  bool grow = false;
  float mb[GT];
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    s[h] = sum_xor32(sum_xor16(s[h]));
    if (valid < 16) s[h] = r < valid ? s[h] : -INFINITY;  // wave uniform
    mb[h] = row_max16(s[h]) * scale_log2;
    grow |= mb[h] > st.m[h] + kRescaleSlack;
  }
  if (__builtin_amdgcn_ballot_w64(grow)) {  // wave-uniform branch, rare after the first blocks
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      const float m_new = mb[h] > st.m[h] + kRescaleSlack ? mb[h] : st.m[h];
      const float alpha = __builtin_amdgcn_exp2f(st.m[h] - m_new);  // 0 when m = -inf, 1 when kept
      st.l[h] *= alpha;
#pragma unroll
      for (int t = 0; t < D / 16; ++t) st.acc[h][t] *= alpha;
      st.m[h] = m_new;
    }
  }
  // the source lanes of this row's tokens 4q, 4q+1 and 4q+2, 4q+3 (bytes)
  const int src01 = (16 * q + 4 * q) * 4, src23 = src01 + 8;
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    const float nm = st.m[h] == -INFINITY ? 0.f : -st.m[h];
    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[h], scale_log2, nm));
    const float pn = dpp_f32<kDppXor1>(p);  // key r ^ 1
    const uint32_t pair = pack_bf16x2(p, pn);  // at even r: keys r (low) and r + 1 (high)
    st.l[h] += __uint_as_float(pair << 16);     // the rounded weight of key r
    const uint32_t w01 = __builtin_amdgcn_ds_bpermute(src01, pair);
    const uint32_t w23 = __builtin_amdgcn_ds_bpermute(src23, pair);
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      const uint2 vh = reinterpret_cast<const uint2*>(&cur.v[t / 2])[t % 2];
      st.acc[h][t] = dot2_bf16(vh.x, w01, st.acc[h][t]);
      st.acc[h][t] = dot2_bf16(vh.y, w23, st.acc[h][t]);
    }
  }
}

// ---------------------------------------------------------------------------
// Split-K over partitions, one contiguous run of partitions per wave.
//
// Units are (sequence, kv head) pairs in sequence-major order; every unit is
// cut into partitions of `partition_tokens` tokens.  The partitions of the
// whole batch, laid end to end, are divided evenly among the waves of a
// persistent grid: wave w takes partitions [w*P/W, (w+1)*P/W).  A wave walks
// the 16-token blocks of its partitions in order, folding consecutive blocks
// (and consecutive partitions) of one unit into one running (m, l, O) state,
// and writes a result only where its run of a unit ends: the final row when
// the unit lies entirely in this wave, else the partial (m, l, O) in slot
// (w + unit), which the merge kernel folds with the same recurrences.  The
// balance is exact for any mix of lengths, and about W + units partials are
// written in total, so the stream of K/V reads is not interleaved with
// per-partition writes.
// ---------------------------------------------------------------------------

// ---------------------------------------------------------------------------
// Multi-query attention as one decode query per chunk row, for the pools the
// multi-query kernel does not read.  Chunk row j of sequence s (c rows,
// context n) sees the keys 0 .. n - c + j ([KVM] chunked prefill mechanism:
// the history and the chunk rows up to its own), so it is a decode query over
// the first n - c + j + 1 keys of s's table.  This kernel writes, per row r,
// that length and the table row to read; the rows of a sequence with
// c > max_q_len or c > n get table row -1 (the decode writes NaN), rows no
// sequence owns get length 0 (a zero row).
// ---------------------------------------------------------------------------

__global__ void __launch_bounds__(256) prefill_rows_kernel(const int32_t* __restrict__ q_indptr,
                                                           const int32_t* __restrict__ ctx, int n_seqs, int total_q,
                                                           int max_q_len, int cap, int32_t* __restrict__ row_len,
                                                           int32_t* __restrict__ row_table) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= total_q) return;
  int len = 0, trow = 0;
  if (n_seqs > 0 && r >= q_indptr[0] && r < q_indptr[n_seqs]) {
    int lo = 0, hi = n_seqs - 1;  // the last sequence whose first row is <= r
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (q_indptr[mid] <= r) lo = mid; else hi = mid - 1;
    }
    const int q0 = q_indptr[lo];
    const int c = q_indptr[lo + 1] - q0;
    const int n = min(ctx[lo], cap);
    const bool bad = c > max_q_len || c > n;
    len = bad ? 1 : n - c + (r - q0) + 1;
    trow = bad ? -1 : lo;
  }
  row_len[r] = len;
  row_table[r] = trow;
}

constexpr int kSkWaves = 4;     // waves per workgroup
constexpr int kSkQUnits = 4;    // at most this many units per wave have staged queries

struct sk_args {
  const void* q;
  void* out;
  const void* k_layer;
  const void* v_layer;
  float* part_m;   // [slots][G]
  float* part_l;   // [slots][G]
  float* part_o;   // [slots][G][D]
  int32_t* cum_parts;  // [n_seqs + 1] partitions before each sequence (written by group 0)
  int n_seqs, max_blocks, n_q_heads, n_kv_heads, num_blocks, part_blocks, n_waves;
  int block_size;  // B: tokens per table entry (the kernel works in 16-token tiles)
  int q_units;  // units per wave whose queries are staged in LDS (<= kSkQUnits)
  float scale_log2;
  // row of the tables that sequence s reads (NULL: row s); a negative row has
  // no valid entry (the sequence's output is NaN)
  const int32_t* table_rows;
};

// LDS ints before the staged queries: cum_b, cum_p (n + 1 each) and ctx_n
// (n), rounded up to 16 bytes.
__host__ __device__ constexpr int sk_prefix_ints(int n_seqs) { return (3 * n_seqs + 2 + 3) & ~3; }


// Exclusive prefix sums, over sequences, of blocks (cum_b) and partitions
// (cum_p), and the clamped context lengths (ctx_n); a workgroup-wide scan in
// LDS, so that the kernel reads the lengths from global memory once.
__device__ __forceinline__ void sk_prefix(const sk_args& a, const int32_t* __restrict__ ctx_lens, int* cum_b,
                                          int* cum_p, int* ctx_n) {
  __shared__ int wsum_b[kSkWaves], wsum_p[kSkWaves];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int cap = a.max_blocks * a.block_size;
  int carry_b = 0, carry_p = 0;
  for (int base = 0; base < a.n_seqs; base += kSkWaves * 64) {
    const int s = base + tid;
    const int n = s < a.n_seqs ? min(ctx_lens[s], cap) : 0;
    const int nb = n > 0 ? (n + 15) >> 4 : 0;
    const int np = (nb + a.part_blocks - 1) / a.part_blocks;
    int ib = nb, ip = np;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int yb = __shfl_up(ib, off), yp = __shfl_up(ip, off);
      if (lane >= off) {
        ib += yb;
        ip += yp;
      }
    }
    if (lane == 63) {
      wsum_b[wv] = ib;
      wsum_p[wv] = ip;
    }
    __syncthreads();
    int before_b = carry_b, before_p = carry_p;
    for (int i = 0; i < wv; ++i) {
      before_b += wsum_b[i];
      before_p += wsum_p[i];
    }
    if (s < a.n_seqs) {
      cum_b[s] = before_b + ib - nb;
      cum_p[s] = before_p + ip - np;
      ctx_n[s] = n;
    }
    for (int i = 0; i < kSkWaves; ++i) {
      carry_b += wsum_b[i];
      carry_p += wsum_p[i];
    }
    __syncthreads();
  }
  if (tid == 0) {
    cum_b[a.n_seqs] = carry_b;
    cum_p[a.n_seqs] = carry_p;
  }
  __syncthreads();
}

// Position of a wave's run in (sequence, kv head, block) terms.  All fields
// are wave uniform.
struct sk_cursor {
  int seq, kvh, j, nb, n, trow;  // trow: the table row of seq
};

// BS is the pool's block size B.  The kernel walks 16-token tiles: for B >= 16
// a table entry holds B/16 tiles (tile j is sub-tile j % (B/16) of entry
// j / (B/16)); for B < 16 a tile gathers 16/B consecutive entries, each lane
// reading its pieces from the entry that holds its keys (K) or its 4 value
// slots (V).  In every case a lane's 16-byte pieces of one tile are exactly its
// matrix operands (the tile layout of the pool puts, for B >= 16, each
// quarter-wave's 16 pieces in one 256-byte run).
// TBL = 1 (bf16, B = 16): the block-table entries of a wave's run are copied
// into an LDS slice of up to kSkTblMax entries when the run starts and read
// from there per tile; 0: one scalar load per tile.
constexpr int kSkTblMax = 2048;

// MATH = 1 (bf16, B = 16): the vector-ALU step attend_block_valu with GT query
// heads per KV head instead of the matrix instructions; 0: matrix instructions.
template <int D, int STAGES, int WAVES_PER_SIMD, int FMT, int BS, int TBL = 0, int MATH = 0, int GT = 1>
__global__ void __launch_bounds__(kSkWaves * 64) __attribute__((amdgpu_waves_per_eu(WAVES_PER_SIMD, WAVES_PER_SIMD)))
attn_mfma_kernel(sk_args a, const int32_t* __restrict__ ctx_lens, const int32_t* __restrict__ tables) {
  static_assert(FMT == kFmtBf16 || BS == 16, "quantised tiles are 16 tokens");
  static_assert(TBL == 0 || (FMT == kFmtBf16 && BS == 16), "LDS-staged table entries: bf16, B = 16");
  static_assert(MATH == 0 || (FMT == kFmtBf16 && BS == 16 && TBL == 0), "vector-ALU step: bf16, B = 16");
  static_assert(BS == 4 || BS == 8 || BS == 16 || BS == 32 || BS == 64, "block size");
  extern __shared__ __align__(16) int sk_smem[];
  int* cum_b = sk_smem;                       // n_seqs + 1
  int* cum_p = sk_smem + a.n_seqs + 1;        // n_seqs + 1
  int* ctx_n = sk_smem + 2 * (a.n_seqs + 1);  // n_seqs
  const int G = a.n_q_heads / a.n_kv_heads;
  const int Hkv = a.n_kv_heads;
  uint16_t* q_s = reinterpret_cast<uint16_t*>(sk_smem + sk_prefix_ints(a.n_seqs));  // [waves][q_units][G][D]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hg = (lane & 15) % G;  // query head (within the group) of this lane's column
  const int quad = lane >> 4;      // 4-token group / 8-dim group of this lane

  sk_prefix(a, ctx_lens, cum_b, cum_p, ctx_n);
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= a.n_seqs; i += kSkWaves * 64) a.cum_parts[i] = cum_p[i];
  // prefix entries are read at wave-uniform addresses; keep them scalar so that
  // every branch below is a scalar branch
  auto cb = [&](int s) { return __builtin_amdgcn_readfirstlane(cum_b[s]); };
  auto cp = [&](int s) { return __builtin_amdgcn_readfirstlane(cum_p[s]); };
  auto cn = [&](int s) { return __builtin_amdgcn_readfirstlane(ctx_n[s]); };

  // this wave's run of partitions
  const int64_t total_parts = static_cast<int64_t>(Hkv) * cp(a.n_seqs);
  const int64_t wid = static_cast<int64_t>(blockIdx.x) * kSkWaves + wave;
  const int64_t p_begin = div_nn(wid * total_parts, a.n_waves);
  const int64_t p_end = div_nn((wid + 1) * total_parts, a.n_waves);
  if (p_begin >= p_end) return;

  // partition index -> (sequence, kv head, first block).  The sequence is the
  // last one whose first partition is <= pp: the lanes test 64 sequences at a
  // time and count the passes (the test holds for a prefix of the sequences).
  auto locate = [&](int64_t pp, sk_cursor& c) {
    int passed = 0;
    for (int base = 0; base < a.n_seqs; base += 64) {
      const int s = base + lane;
      const bool ok = s < a.n_seqs && static_cast<int64_t>(Hkv) * cum_p[s] <= pp;
      const uint64_t m = __builtin_amdgcn_ballot_w64(ok);
      passed += __builtin_popcountll(m);
      if (m != ~0ull) break;
    }
    const int lo = max(passed - 1, 0);
    c.seq = lo;
    const int np = cp(lo + 1) - cp(lo);
    const int64_t r = pp - static_cast<int64_t>(Hkv) * cp(lo);
    const int64_t h = div_nn(r, np);
    c.kvh = static_cast<int>(h);
    c.j = static_cast<int>(r - h * np) * a.part_blocks;
    c.nb = cb(lo + 1) - cb(lo);
    c.n = cn(lo);
    c.trow = a.table_rows ? a.table_rows[lo] : lo;
  };
  sk_cursor first, last;
  locate(p_begin, first);
  locate(p_end - 1, last);
  last.j = min(last.j + a.part_blocks, last.nb) - 1;
  auto flat = [&](const sk_cursor& c) -> int64_t {
    return static_cast<int64_t>(Hkv) * cb(c.seq) + static_cast<int64_t>(c.kvh) * c.nb + c.j;
  };
  const int n_blk = static_cast<int>(flat(last) - flat(first)) + 1;  // blocks of this run

  // step a cursor to the next block of the run
  auto advance = [&](sk_cursor& c) {
    if (++c.j < c.nb) return;
    c.j = 0;
    if (++c.kvh < Hkv) return;
    c.kvh = 0;
    do {
      ++c.seq;
    } while (c.seq < a.n_seqs - 1 && cb(c.seq + 1) == cb(c.seq));
    c.nb = cb(c.seq + 1) - cb(c.seq);
    c.n = cn(c.seq);
    c.trow = a.table_rows ? ((const __attribute__((address_space(4))) int32_t*)a.table_rows)[c.seq] : c.seq;
  };

  // TBL = 1: the table entries of the run's first tbl_n blocks, block k of the
  // run at tbl_wave[k].  The lanes copy consecutive entries of each unit of
  // the run straight from global memory into the slice (no registers), and
  // the wave waits for them once, before the ring is first filled.
  int* tbl_wave = nullptr;
  int tbl_n = 0;
  if constexpr (TBL != 0) {
    tbl_wave = reinterpret_cast<int*>(q_s + static_cast<int64_t>(kSkWaves) * a.q_units * G * D) + wave * kSkTblMax;
    tbl_n = min(n_blk, kSkTblMax);
    sk_cursor c = first;
    for (int k0 = 0; k0 < tbl_n;) {
      const int cnt = min(c.nb - c.j, tbl_n - k0);  // the unit's blocks in the staged part of the run
      for (int i = 0; i < cnt; i += 64) {
        if (lane < cnt - i) {
          if (c.trow >= 0) {
            const int32_t* src = tables + static_cast<int64_t>(c.trow) * a.max_blocks + c.j + i + lane;
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src),
                                             (__attribute__((address_space(3))) void*)(tbl_wave + k0 + i), 4, 0, 0);
          } else {
            tbl_wave[k0 + i + lane] = -1;  // a row without valid entries
          }
        }
      }
      k0 += cnt;
      if (k0 < tbl_n) {
        c.j = c.nb - 1;
        advance(c);  // the next unit
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // every counter: the copies and the stores have landed
  }

  // ring entries: bf16 operand tiles, or raw quantised tiles (codes and scales) converted on use
  using ring_t = typename std::conditional<FMT == kFmtBf16, kv_regs<D>, kv_qregs<D, FMT>>::type;
  const uint4* kpool = static_cast<const uint4*>(a.k_layer);
  const uint4* vpool = static_cast<const uint4*>(a.v_layer);

  // load side: the tile STAGES ahead of consumption (the last one repeats
  // past the end of the run and is served by the L2)
  sk_cursor ld = first;
  int ld_k = 0;
  bool bad_ring[STAGES];  // a table entry the tile needs lies outside [0, N)
  // Lane offsets, in 16-byte pieces inside a (block, kv head) tile of BS * D
  // elements, of the lane's first K and V piece; its i-th piece is 4 BS pieces
  // further.  With r = lane % 16, a lane holds key r and, for V, value slots
  // 4 quad .. 4 quad + 3 of the 16-token tile.
  constexpr int64_t kEntryVec = static_cast<int64_t>(BS) * D * 2 / 16;
  const int k_lane = quad * BS + (BS >= 16 ? (lane & 15) : (lane & 15) % BS);
  const int v_lane = BS >= 16 ? lane : ((quad * 4) % BS / 4) * 16 + (lane & 15);
  auto issue = [&](ring_t& buf, int u) {
    const int64_t row = static_cast<int64_t>(ld.trow) * a.max_blocks;
    if constexpr (FMT != kFmtBf16) {
      const int phys = ld.trow >= 0 ? tables[row + ld.j] : -1;
      const bool bad = phys < 0 || phys >= a.num_blocks;
      bad_ring[u] = bad;
      const int p = bad ? 0 : phys;  // never dereferenced out of range
      const int64_t t = (static_cast<int64_t>(p) * Hkv + ld.kvh) * q_tile_bytes<D, FMT>();
      load_qblock<D, FMT>(buf, static_cast<const unsigned char*>(a.k_layer) + t,
                          static_cast<const unsigned char*>(a.v_layer) + t, lane);
    } else if constexpr (BS >= 16) {
      // tile j is sub-tile j % (BS/16) of entry j / (BS/16)
      constexpr int kSub = BS / 16;
      // (the table through the constant address space: after the copies into
      // LDS the compiler would otherwise turn these uniform reads into vector
      // loads, whose waits drain the ring)
      int phys;
      if (TBL != 0 && ld_k < tbl_n)
        phys = __builtin_amdgcn_readfirstlane(tbl_wave[ld_k]);
      else
        phys = ld.trow >= 0 ? ((const __attribute__((address_space(4))) int32_t*)tables)[row + ld.j / kSub] : -1;
      const bool bad = phys < 0 || phys >= a.num_blocks;
      bad_ring[u] = bad;
      const int p = bad ? 0 : phys;
      const int sub = ld.j % kSub;
      const int64_t t = (static_cast<int64_t>(p) * Hkv + ld.kvh) * kEntryVec;
      load_block_strided<D, 4 * BS>(buf, kpool + t + sub * 16 + k_lane, vpool + t + sub * 64 + v_lane);
    } else {
      // tile j gathers entries j * (16/BS) + e; only those holding tokens of
      // the context are read (the others may lie past the table's row)
      constexpr int kPer = 16 / BS;
      int phys[kPer];
      bool bad = false;
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        const bool needed = ld.j * 16 + e * BS < ld.n;
        const int ph = !needed ? 0 : (ld.trow >= 0 ? tables[row + ld.j * kPer + e] : -1);
        const bool b = ph < 0 || ph >= a.num_blocks;
        bad |= b;
        phys[e] = b ? 0 : ph;
      }
      bad_ring[u] = bad;
      int pk = phys[0], pv = phys[0];
#pragma unroll
      for (int e = 1; e < kPer; ++e) {
        pk = (lane & 15) / BS == e ? phys[e] : pk;
        pv = quad * 4 / BS == e ? phys[e] : pv;
      }
      load_block_strided<D, 4 * BS>(buf, kpool + (static_cast<int64_t>(pk) * Hkv + ld.kvh) * kEntryVec + k_lane,
                                    vpool + (static_cast<int64_t>(pv) * Hkv + ld.kvh) * kEntryVec + v_lane);
    }
    if (++ld_k < n_blk) advance(ld);
  };

  ring_t buf[STAGES];
#pragma unroll
  for (int u = 0; u < STAGES; ++u) issue(buf[u], u);

  // stage the queries of the first q_units units of the run in LDS (issued
  // after the first ring loads, so that both wait out one memory latency)
  uint16_t* q_wave = q_s + static_cast<int64_t>(wave) * a.q_units * G * D;
  {
    sk_cursor c = first;
    for (int i = 0; i < a.q_units; ++i) {
      const uint16_t* qg = static_cast<const uint16_t*>(a.q) +
                           (static_cast<int64_t>(c.seq) * a.n_q_heads + c.kvh * G) * D;
      for (int e = lane * 8; e < G * D; e += 64 * 8)
        *reinterpret_cast<uint4*>(q_wave + i * G * D + e) = *reinterpret_cast<const uint4*>(qg + e);
      if (c.seq == last.seq && c.kvh == last.kvh) break;
      // next unit
      c.j = c.nb - 1;
      advance(c);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // consume side
  sk_cursor cs = first;
  int unit_idx = 0;   // index of the current unit within the run
  int seg_j0 = first.j;
  bf16x8_t qop[D / 32];
  f32x4_t kbias[D / 32];  // q4_0: the score accumulators' start (zeros otherwise)
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) kbias[kk] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // queries of the idx-th unit of the run: always read from LDS (a unit past
  // the staged ones is first copied into the slot of an earlier, finished
  // unit), so the query registers never wait on global loads in the loop
  int q_slot = 0;  // LDS slot of the current unit's queries
  auto fetch_q = [&](int idx) {
    const int slot = idx % a.q_units;
    q_slot = slot;
    if (idx >= a.q_units) {
      const uint16_t* qg = static_cast<const uint16_t*>(a.q) +
                           (static_cast<int64_t>(cs.seq) * a.n_q_heads + cs.kvh * G) * D;
      for (int e = lane * 8; e < G * D; e += 64 * 8)
        *reinterpret_cast<uint4*>(q_wave + slot * G * D + e) = *reinterpret_cast<const uint4*>(qg + e);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
      qop[kk] = *reinterpret_cast<const bf16x8_t*>(q_wave + slot * G * D + hg * D + kk * 32 + quad * 8);
    if constexpr (FMT == kFmtQ4) {  // -kQ4Bias times the query's sum over each group (all four quads)
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        const uint4 w = __builtin_bit_cast(uint4, qop[kk]);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
        float part = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) part += __uint_as_float(ws[k] << 16) + __uint_as_float(ws[k] & 0xffff0000u);
        const float b = -kQ4Bias * sum_xor32(sum_xor16(part));
        kbias[kk] = f32x4_t{b, b, b, b};
      }
    }
  };
  fetch_q(0);

  f32x4_t o[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_lane = 0.f;
  bool poisoned = false;

  // vector-ALU step: its own state and result layout (lane (r, q) ends with
  // O[h][16 t + r] for every head once the quads are added; quad q writes the
  // tiles t = 2q, 2q + 1 of D = 128, in general t = q, q + 4, ...)
  valu_state<D, GT> vst;
  if constexpr (MATH == 1) valu_reset(vst);
  auto finish_valu = [&]() {
    const int r = lane & 15;
    const float nan = __builtin_nanf("");
    const bool whole = seg_j0 == 0 && cs.j == cs.nb - 1;
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      const float l = row_sum16(vst.l[h]);
      const int head = cs.kvh * G + h;
      float* po = nullptr;
      uint16_t* orow = nullptr;
      const int64_t prow = (wid + static_cast<int64_t>(cs.seq) * Hkv + cs.kvh) * G + h;
      if (whole)
        orow = static_cast<uint16_t*>(a.out) + (static_cast<int64_t>(cs.seq) * a.n_q_heads + head) * D;
      else
        po = a.part_o + prow * D;
      const float inv = poisoned ? 0.f : 1.f / l;
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        const float v = sum_xor32(sum_xor16(vst.acc[h][t]));
        if (t % 4 != quad) continue;
        if (whole)
          orow[16 * t + r] = poisoned ? static_cast<uint16_t>(0x7fc0) : f32_to_bf16(v * inv);
        else
          po[16 * t + r] = poisoned ? nan : v;
      }
      if (!whole && lane == 0) {
        a.part_m[prow] = poisoned ? nan : vst.m[h];
        a.part_l[prow] = poisoned ? nan : l;
      }
    }
    valu_reset(vst);
    poisoned = false;
  };

  // writes the result of the current unit's run and resets the state
  auto finish = [&]() {
    if constexpr (MATH == 1) {
      finish_valu();
      return;
    }
    const float l = sum_xor32(sum_xor16(l_lane));
    const int h = cs.kvh * G + hg;
    const float nan = __builtin_nanf("");
    if (seg_j0 == 0 && cs.j == cs.nb - 1) {  // the whole unit: final row
      const float inv = poisoned ? 0.f : 1.f / l;
      uint16_t* out = static_cast<uint16_t*>(a.out) + (static_cast<int64_t>(cs.seq) * a.n_q_heads + h) * D;
#pragma unroll
      for (int nt = 0; nt < D / 16; ++nt) {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = poisoned ? nan : o[nt][i] * inv;
        *reinterpret_cast<uint2*>(out + nt * 16 + quad * 4) =
            make_uint2(static_cast<uint32_t>(f32_to_bf16(v[0])) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16),
                       static_cast<uint32_t>(f32_to_bf16(v[2])) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16));
      }
    } else {
      const int64_t slot = wid + static_cast<int64_t>(cs.seq) * Hkv + cs.kvh;
      const int64_t row = slot * G + hg;
      float* po = a.part_o + row * D;
#pragma unroll
      for (int nt = 0; nt < D / 16; ++nt)
        *reinterpret_cast<float4*>(po + nt * 16 + quad * 4) =
            poisoned ? make_float4(nan, nan, nan, nan) : make_float4(o[nt][0], o[nt][1], o[nt][2], o[nt][3]);
      a.part_m[row] = poisoned ? nan : m_run;
      a.part_l[row] = poisoned ? nan : l;
    }
#pragma unroll
    for (int i = 0; i < D / 16; ++i) o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m_run = -INFINITY;
    l_lane = 0.f;
    poisoned = false;
  };

  // STAGES-deep register ring: block k lives in buf[k % STAGES]; every slot is
  // refilled right after it is consumed, so STAGES-1 blocks stay in flight.
  int k0 = 0;
  do {
#pragma unroll
    for (int u = 0; u < STAGES; ++u) {
      const int k = k0 + u;
      if (k < n_blk) {
        const bool bad = bad_ring[u];
        poisoned |= bad;
        const int valid = bad ? 0 : min(16, cs.n - cs.j * 16);
        if constexpr (MATH == 1) {
          attend_block_valu<D, GT>(buf[u], q_wave + q_slot * G * D, valid, lane, a.scale_log2, vst);
        } else if constexpr (FMT == kFmtBf16) {
          attend_block<D>(buf[u], qop, valid, quad, a.scale_log2, o, m_run, l_lane);
        } else {
          kv_regs<D> tile;
          codes_block<D, FMT>(buf[u], tile);
          attend_qblock<D, FMT>(tile, buf[u], qop, kbias, valid, quad, a.scale_log2, o, m_run, l_lane);
        }
        if (cs.j == cs.nb - 1 || k == n_blk - 1) {  // end of this unit's run
          finish();
          if (k + 1 < n_blk) {
            advance(cs);
            seg_j0 = 0;
            fetch_q(++unit_idx);
          }
        } else {
          advance(cs);
        }
      }
      issue(buf[u], u);
    }
    k0 += STAGES;
  } while (k0 < n_blk);
}

// Merge for the split-K kernel: unit (seq, kv head) was covered by waves
// wF..wL (the waves whose runs hold its first and last partition); unless one
// wave held it whole, fold the partials of slots w + unit with the
// running-max recurrences.  Also writes zero rows for empty sequences.  One
// wave per (sequence, query head), four per workgroup: lane p holds the weight
// of partial p (64 at a time) and every lane then accumulates its D/64 dims
// over the partials, four row loads in flight.
constexpr int kMergeItems = 4;
constexpr int kMergeFast = 8;  // partials per item loaded all at once

template <int D>
__global__ void __launch_bounds__(kMergeItems * 64) merge_sk_kernel(sk_args a) {
  constexpr int E = D / 64;  // dims per lane
  const int lane = threadIdx.x & 63;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * kMergeItems + (threadIdx.x >> 6);
  if (item >= static_cast<int64_t>(a.n_seqs) * a.n_q_heads) return;
  const int seq = static_cast<int>(item / a.n_q_heads);
  const int h = static_cast<int>(item % a.n_q_heads);
  const int G = a.n_q_heads / a.n_kv_heads;
  const int kvh = h / G, hg = h % G;
  uint16_t* out = static_cast<uint16_t*>(a.out) + item * D + lane * E;
  const int np = a.cum_parts[seq + 1] - a.cum_parts[seq];
  if (np == 0) {
#pragma unroll
    for (int j = 0; j < E; ++j) out[j] = 0;
    return;
  }
  const int64_t total = static_cast<int64_t>(a.n_kv_heads) * a.cum_parts[a.n_seqs];
  const int64_t W = a.n_waves;
  const int64_t first = static_cast<int64_t>(a.n_kv_heads) * a.cum_parts[seq] + static_cast<int64_t>(kvh) * np;
  auto wave_of = [&](int64_t pp) { return div_nn((pp + 1) * W - 1, total); };
  auto run_begin = [&](int64_t w) { return div_nn(w * total, W); };
  const int64_t wF = wave_of(first), wL = wave_of(first + np - 1);
  if (wF == wL) return;  // one wave wrote the final row
  const int n_w = static_cast<int>(wL - wF + 1);
  const int64_t unit = static_cast<int64_t>(seq) * a.n_kv_heads + kvh;
  auto row_of = [&](int i) { return (wF + i + unit) * G + hg; };
  auto live = [&](int i) { return run_begin(wF + i) < run_begin(wF + i + 1); };
  auto load_row = [&](int i, float (&v)[E]) {
    const float* o = a.part_o + row_of(i) * D + lane * E;
    if constexpr (E == 4) {
      const float4 t = *reinterpret_cast<const float4*>(o);
      v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    } else if constexpr (E == 2) {
      const float2 t = *reinterpret_cast<const float2*>(o);
      v[0] = t.x; v[1] = t.y;
    } else {
      v[0] = o[0];
    }
  };
  if (n_w <= kMergeFast) {
    // few partials (the usual case): every load of the item is issued at
    // once -- each lane's (m, l) and all rows -- so the merge waits out one
    // memory latency after the prefix read
    float m = -INFINITY, l = 0.f;
    if (lane < n_w && live(lane)) {
      m = a.part_m[row_of(lane)];
      l = a.part_l[row_of(lane)];
    }
    float v[kMergeFast][E];
#pragma unroll
    for (int k = 0; k < kMergeFast; ++k)
      if (k < n_w && live(k)) load_row(k, v[k]);
    const bool nan = __builtin_amdgcn_ballot_w64(m != m) != 0;
    const float M = wave_max(m != m ? -INFINITY : m);
    const float w = (m != m) ? 0.f : __builtin_amdgcn_exp2f(m - M);
    const float L = wave_sum(w * l);
    float acc[E];
#pragma unroll
    for (int j = 0; j < E; ++j) acc[j] = 0.f;
#pragma unroll
    for (int k = 0; k < kMergeFast; ++k) {
      const float wk = __shfl(w, k);
      if (k < n_w && wk != 0.f)
#pragma unroll
        for (int j = 0; j < E; ++j) acc[j] = __builtin_fmaf(wk, v[k][j], acc[j]);
    }
    const float inv = 1.f / L;
#pragma unroll
    for (int j = 0; j < E; ++j) out[j] = nan ? static_cast<uint16_t>(0x7fc0) : f32_to_bf16(acc[j] * inv);
    return;
  }
  float M = -INFINITY;
  bool nan = false;
  for (int i = lane; i < n_w; i += 64)
    if (live(i)) {
      const float m = a.part_m[row_of(i)];
      nan |= m != m;
      M = fmaxf(M, m);
    }
  M = wave_max(M);
  nan = __builtin_amdgcn_ballot_w64(nan) != 0;
  float acc[E];
#pragma unroll
  for (int j = 0; j < E; ++j) acc[j] = 0.f;
  float L = 0.f;
  for (int i0 = 0; i0 < n_w; i0 += 64) {
    float w = 0.f;
    if (i0 + lane < n_w && live(i0 + lane)) {
      const float m = a.part_m[row_of(i0 + lane)];
      w = (m != m) ? 0.f : __builtin_amdgcn_exp2f(m - M);
      L += w * a.part_l[row_of(i0 + lane)];
    }
    const int cnt = min(64, n_w - i0);
#pragma unroll 4
    for (int k = 0; k < cnt; ++k) {
      const float wk = __shfl(w, k);
      const float* o = a.part_o + row_of(i0 + k) * D + lane * E;
      float v[E];
      if constexpr (E == 4) {
        const float4 t = *reinterpret_cast<const float4*>(o);
        v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
      } else if constexpr (E == 2) {
        const float2 t = *reinterpret_cast<const float2*>(o);
        v[0] = t.x; v[1] = t.y;
      } else {
        v[0] = o[0];
      }
#pragma unroll
      for (int j = 0; j < E; ++j) acc[j] = wk == 0.f ? acc[j] : __builtin_fmaf(wk, v[j], acc[j]);
    }
  }
  L = wave_sum(L);
  const float inv = 1.f / L;
#pragma unroll
  for (int j = 0; j < E; ++j) out[j] = nan ? static_cast<uint16_t>(0x7fc0) : f32_to_bf16(acc[j] * inv);
}

// ---------------------------------------------------------------------------
// Merge of the partitions of a sequence with the running-max recurrences:
// M = max_p m_p, out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p.
// One workgroup per (sequence, query head); sequences with one partition were
// finished by the partition kernel.
// ---------------------------------------------------------------------------

constexpr int kMergeThreads = 256;
constexpr int kMergeWeights = 2048;  // partitions whose weights are kept in LDS

template <typename T>
__global__ void __launch_bounds__(kMergeThreads) merge_kernel(attn_args a) {
  const int seq = blockIdx.x / a.n_q_heads;
  const int h = blockIdx.x % a.n_q_heads;
  int n = a.ctx_lens[seq];
  const int cap = a.max_blocks * a.block_size;
  n = n > cap ? cap : n;
  const int n_parts = n <= 0 ? 1 : (n + a.partition_tokens - 1) / a.partition_tokens;
  if (n_parts == 1) return;
  const int64_t ph = (static_cast<int64_t>(seq) * a.n_q_heads + h) * a.max_parts;
  __shared__ float w_s[kMergeWeights];
  __shared__ float red[kMergeThreads / 64];
  __shared__ float4 acc_s[kMergeThreads];
  const int tid = threadIdx.x;
  // maximum over partitions
  float M = -INFINITY;
  for (int p = tid; p < n_parts; p += kMergeThreads) M = fmaxf(M, a.part_m[ph + p]);
  M = wave_max(M);
  if ((tid & 63) == 0) red[tid >> 6] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  // weights 2^(m_p - M) and the denominator
  float L = 0.f;
  for (int p = tid; p < n_parts; p += kMergeThreads) {
    const float m = a.part_m[ph + p];
    const float f = (m != m) ? __builtin_nanf("") : exp2f(m - M);
    if (p < kMergeWeights) w_s[p] = f;
    L += f * a.part_l[ph + p];
  }
  L = wave_sum(L);
  if ((tid & 63) == 0) red[tid >> 6] = L;
  __syncthreads();
  L = red[0] + red[1] + red[2] + red[3];
  // weighted sum of the partial outputs: each thread owns 4 dims of every
  // groups-th partition, 16-byte loads
  const int d4 = a.head_dim / 4;
  const int groups = kMergeThreads / d4;
  const int grp = tid / d4, c = tid % d4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (grp < groups) {
    for (int p = grp; p < n_parts; p += groups) {
      const float f = p < kMergeWeights ? w_s[p] : exp2f(a.part_m[ph + p] - M);
      const float4 v = reinterpret_cast<const float4*>(a.part_o + (ph + p) * a.head_dim)[c];
      acc.x += f * v.x;
      acc.y += f * v.y;
      acc.z += f * v.z;
      acc.w += f * v.w;
    }
  }
  acc_s[tid] = acc;
  __syncthreads();
  if (tid < d4) {
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int g = 0; g < groups; ++g) {
      const float4 v = acc_s[g * d4 + tid];
      sum.x += v.x;
      sum.y += v.y;
      sum.z += v.z;
      sum.w += v.w;
    }
    const float inv = 1.f / L;
    T* out = static_cast<T*>(a.out) + (static_cast<int64_t>(seq) * a.n_q_heads + h) * a.head_dim + 4 * tid;
    out[0] = elem<T>::from_f32(sum.x * inv);
    out[1] = elem<T>::from_f32(sum.y * inv);
    out[2] = elem<T>::from_f32(sum.z * inv);
    out[3] = elem<T>::from_f32(sum.w * inv);
  }
}

// ---------------------------------------------------------------------------
// host helpers
// ---------------------------------------------------------------------------

}  // namespace

kv_status hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return KV_OK;
  return fail(KV_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool mfma_supported(const kv_pool_config& c, int G) {
  return (c.dtype == KV_BF16 || is_quantized(c.dtype)) && c.block_size == 16 &&
         (c.head_dim == 64 || c.head_dim == 128 || c.head_dim == 256) && G >= 1 && G <= kMaxGroup;
}

// The split-K decode kernel also reads bf16 pools of block size 4, 8, 32, 64.
bool decode_mfma_supported(const kv_pool_config& c, int G) {
  if (mfma_supported(c, G)) return true;
  const int b = c.block_size;
  return c.dtype == KV_BF16 && (b == 4 || b == 8 || b == 32 || b == 64) &&
         (c.head_dim == 64 || c.head_dim == 128 || c.head_dim == 256) && G >= 1 && G <= kMaxGroup;
}

int device_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
  }
  return cus;
}

// LDS a workgroup may use on the current device.
size_t max_lds_per_block() {
  static int bytes = -1;
  if (bytes < 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&bytes, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || bytes < 0)
      bytes = 65536;
  }
  return static_cast<size_t>(bytes);
}

uint64_t up256(uint64_t b) { return (b + 255) & ~uint64_t(255); }

namespace {

// Partition length of the generic kernel: aim for a few thousand workgroups
// so every CU has several resident, at least 256 tokens each.
int choose_generic_partition(const kv_pool_config& c, int n_seqs, int max_blocks) {
  const int64_t max_ctx = static_cast<int64_t>(max_blocks) * c.block_size;
  const int64_t units = static_cast<int64_t>(n_seqs) * c.num_kv_heads;
  int part = 16 * c.block_size;
  while (part < max_ctx && units * ((max_ctx + part - 1) / part) > 4096) part *= 2;
  return part;
}

// The split-K kernel keeps, per workgroup, two prefix arrays over sequences
// and the staged queries in LDS.
constexpr int kSkMaxSeqs = 4095;
constexpr int kSkQBudget = 8192;  // bytes of staged queries per wave

// Units per wave with staged queries: up to kSkQUnits within the per-wave
// budget and what the prefix arrays leave of the workgroup's LDS; 0 when not
// even one unit fits (then the kernel cannot run).
int sk_q_units(int n_seqs, int G, int D) {
  const int64_t unit = static_cast<int64_t>(G) * D * 2;
  const int64_t left = static_cast<int64_t>(max_lds_per_block()) - static_cast<int64_t>(sk_prefix_ints(n_seqs)) * 4;
  const int64_t fit = left > 0 ? left / (kSkWaves * unit) : 0;
  return static_cast<int>(std::min<int64_t>({kSkQUnits, std::max<int64_t>(1, kSkQBudget / unit), fit}));
}

size_t sk_lds_bytes(int n_seqs, int G, int D) {
  const size_t prefix = static_cast<size_t>(sk_prefix_ints(n_seqs)) * 4;
  return prefix + static_cast<size_t>(kSkWaves) * sk_q_units(n_seqs, G, D) * G * D * 2;
}

// One wave per SIMD.  With two, the scheduler's oldest-first issue lets one
// wave of each pair stream ~1.6x faster than the other; with equal shares the
// slower half then finishes alone with half the loads in flight.  A single
// wave per SIMD with a deeper ring keeps the same bytes in flight per CU.
constexpr int fmt_of(int32_t dtype) { return dtype == KV_Q8_0 ? kFmtQ8 : (dtype == KV_Q4_0 ? kFmtQ4 : kFmtBf16); }

// Waves per SIMD and register-ring depth (blocks in flight per wave).  bf16:
// one wave per SIMD with a deep ring (the waves of one SIMD are issued oldest
// first, so two waves with equal shares finish far apart).  Quantised: code
// conversion and scaling are vector-ALU work that one wave cannot overlap with
// its own loads; two waves per SIMD with a shorter ring measured 1.25-1.4x faster.
constexpr int sk_waves_per_simd(int D, int fmt) { return fmt != kFmtBf16 && D < 256 ? 2 : 1; }

template <int D, int FMT>
constexpr int sk_stages() {
  return D >= 256 ? 2 : (FMT == kFmtBf16 ? 6 : 4);
}

struct resolved {
  int kernel;
  bool staged_table = false;  // KV_KERNEL_MFMA_STAGED_TABLE (kernel is then KV_KERNEL_MFMA)
  bool valu = false;          // KV_KERNEL_VALU (kernel is then KV_KERNEL_MFMA)
  int partition;   // tokens
  int max_parts;   // generic kernel: partitions of the longest context
  int64_t groups;  // split-K kernel: persistent workgroups
  float scale;
};

kv_status resolve(const kv_pool* pool, int n_seqs, int num_q_heads, int max_blocks, const kv_attention_options* opts,
                  resolved& r) {
  const kv_pool_config& c = pool->cfg;
  if (num_q_heads <= 0 || num_q_heads % c.num_kv_heads != 0)
    return fail(KV_ERR_INVALID, "num_q_heads must be a positive multiple of num_kv_heads");
  const int G = num_q_heads / c.num_kv_heads;
  if (G > kMaxGroup) return fail(KV_ERR_UNSUPPORTED, "more than 16 query heads per KV head");
  if (n_seqs < 0 || max_blocks <= 0) return fail(KV_ERR_INVALID, "n_seqs must be >= 0 and max_blocks_per_seq > 0");
  kv_attention_options o{0.f, 0, KV_KERNEL_AUTO, nullptr};
  if (opts) o = *opts;
  if (o.kernel != KV_KERNEL_AUTO && o.kernel != KV_KERNEL_GENERIC && o.kernel != KV_KERNEL_MFMA &&
      o.kernel != KV_KERNEL_MFMA_STAGED_TABLE && o.kernel != KV_KERNEL_VALU)
    return fail(KV_ERR_INVALID, "unknown kernel selector");
  r.valu = o.kernel == KV_KERNEL_VALU;
  if (r.valu) {
    if (c.dtype != KV_BF16 || c.block_size != 16 || c.head_dim != 128 || (G != 4 && G != 8))
      return fail(KV_ERR_UNSUPPORTED, "the vector-ALU split-K kernel reads bf16 pools with B = 16, d = 128, "
                                      "G = 4 or 8");
    o.kernel = KV_KERNEL_MFMA;
  }
  r.staged_table = o.kernel == KV_KERNEL_MFMA_STAGED_TABLE;
  if (r.staged_table) {
    if (c.dtype != KV_BF16 || c.block_size != 16)
      return fail(KV_ERR_UNSUPPORTED, "the LDS-staged table variant reads bf16 pools with B = 16");
    o.kernel = KV_KERNEL_MFMA;
  }
  // a batch of more than kSkMaxSeqs sequences runs as consecutive launches of
  // at most kSkMaxSeqs (the kernel keeps per-sequence prefix sums in LDS)
  const int launch_seqs = std::min(n_seqs, kSkMaxSeqs);
  const bool mfma_ok = decode_mfma_supported(c, G) && sk_q_units(launch_seqs, G, c.head_dim) >= 1;
  if (r.staged_table &&
      (!mfma_ok || sk_lds_bytes(launch_seqs, G, c.head_dim) + kSkWaves * kSkTblMax * 4 > max_lds_per_block()))
    return fail(KV_ERR_UNSUPPORTED, "the LDS-staged table variant does not fit this call");
  if (o.kernel == KV_KERNEL_MFMA && !mfma_ok)
    return fail(KV_ERR_UNSUPPORTED,
                "the matrix-core kernel needs bf16 with B in {4, 8, 16, 32, 64} or q8_0/q4_0 with B = 16, d in "
                "{64, 128, 256}");
  if (is_quantized(c.dtype) && (o.kernel == KV_KERNEL_GENERIC || !mfma_ok))
    return fail(KV_ERR_UNSUPPORTED, "a quantised pool is read by the matrix-core kernel only (G <= 16)");
  r.kernel = o.kernel == KV_KERNEL_AUTO ? (mfma_ok ? KV_KERNEL_MFMA : KV_KERNEL_GENERIC) : o.kernel;
  if (o.partition_tokens < 0 || (o.partition_tokens > 0 && o.partition_tokens % c.block_size != 0))
    return fail(KV_ERR_INVALID, "partition_tokens must be 0 or a positive multiple of the block size");
  if (!(o.scale >= 0.f) || std::isinf(o.scale)) return fail(KV_ERR_INVALID, "scale must be finite and >= 0");
  r.scale = o.scale > 0.f ? o.scale : 1.f / std::sqrt(static_cast<float>(c.head_dim));
  const int64_t max_ctx = static_cast<int64_t>(max_blocks) * c.block_size;
  if (r.kernel == KV_KERNEL_MFMA) {
    // default: one 16-token tile per partition, the finest split (exact
    // balance); a requested length is rounded up to whole tiles
    r.partition = o.partition_tokens ? (o.partition_tokens + 15) / 16 * 16 : 16;
    r.max_parts = static_cast<int>((max_ctx + r.partition - 1) / r.partition);
    const int64_t parts_ub = static_cast<int64_t>(n_seqs) * c.num_kv_heads * r.max_parts;
    r.groups = std::max<int64_t>(
        1, std::min<int64_t>((parts_ub + kSkWaves - 1) / kSkWaves, sk_waves_per_simd(c.head_dim, fmt_of(c.dtype)) * device_cus()));
  } else {
    r.partition = o.partition_tokens ? o.partition_tokens : choose_generic_partition(c, n_seqs, max_blocks);
    r.max_parts = static_cast<int>((max_ctx + r.partition - 1) / r.partition);
    r.groups = 0;
  }
  return KV_OK;
}

// Workspace layout.  Generic kernel: m, l [n_seqs][Hq][max_parts], o [..][d].
// Split-K kernel: m, l [slots][G], o [slots][G][d], slots = waves + units,
// then the partition prefix [n_seqs + 1].
uint64_t workspace_for(const kv_pool_config& c, int n_seqs, int num_q_heads, const resolved& r) {
  if (r.kernel == KV_KERNEL_MFMA) {  // one launch's worth: at most kSkMaxSeqs sequences
    const int G = num_q_heads / c.num_kv_heads;
    const int n = std::min(n_seqs, kSkMaxSeqs);
    const uint64_t slots = static_cast<uint64_t>(r.groups) * kSkWaves + static_cast<uint64_t>(n) * c.num_kv_heads;
    return 2 * up256(slots * G * 4) + up256(slots * G * c.head_dim * 4) + up256((n + 1) * 4ull);
  }
  if (r.max_parts <= 1) return 0;
  const uint64_t rows = static_cast<uint64_t>(n_seqs) * num_q_heads * r.max_parts;
  return up256(rows * 4) * 2 + up256(rows * c.head_dim * 4);
}

template <int D, int FMT, int BS = 16>
hipError_t launch_mfma(const sk_args& a, const int32_t* ctx_lens, const int32_t* tables, int64_t groups, int G,
                       hipStream_t st, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr, bool staged_table = false,
                       bool valu = false) {
  constexpr int kStages = sk_stages<D, FMT>();
  constexpr int kWps = sk_waves_per_simd(D, FMT);
  if constexpr (FMT == kFmtBf16 && BS == 16 && D == 128) {
    // the vector-ALU variant: a 4-deep ring (3 at G = 8) beside its G x D / 16 accumulators per lane
    const uint32_t lds = static_cast<uint32_t>(sk_lds_bytes(a.n_seqs, G, D));
    if (valu && G == 4)
      return launch_timed(attn_mfma_kernel<D, 4, 1, FMT, BS, 0, 1, 4>, dim3(static_cast<unsigned>(groups)),
                          dim3(kSkWaves * 64), lds, st, ev0, ev1, a, ctx_lens, tables);
    if (valu && G == 8)
      return launch_timed(attn_mfma_kernel<D, 3, 1, FMT, BS, 0, 1, 8>, dim3(static_cast<unsigned>(groups)),
                          dim3(kSkWaves * 64), lds, st, ev0, ev1, a, ctx_lens, tables);
  }
  if (valu) return hipErrorInvalidValue;
  if constexpr (FMT == kFmtBf16 && BS == 16) {
    if (staged_table)
      return launch_timed(attn_mfma_kernel<D, kStages, kWps, FMT, BS, 1>, dim3(static_cast<unsigned>(groups)),
                          dim3(kSkWaves * 64),
                          static_cast<uint32_t>(sk_lds_bytes(a.n_seqs, G, D) + kSkWaves * kSkTblMax * 4), st, ev0,
                          ev1, a, ctx_lens, tables);
  }
  return launch_timed(attn_mfma_kernel<D, kStages, kWps, FMT, BS>, dim3(static_cast<unsigned>(groups)),
                      dim3(kSkWaves * 64), static_cast<uint32_t>(sk_lds_bytes(a.n_seqs, G, D)), st, ev0, ev1, a,
                      ctx_lens, tables);
}

template <typename T, int D>
hipError_t launch_generic(const attn_args& a, int64_t grid, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  return launch_timed(attn_generic_kernel<T, D>, dim3(static_cast<unsigned>(grid)), dim3(256), 0u, st, ev0, ev1, a);
}

// The decode kernels and their merge for arguments already checked.  Sequence
// s reads row table_rows[s] of the tables (row s when table_rows is NULL).
kv_status decode_launch(const kv_pool* pool, int layer, const void* q, void* out, const int32_t* d_block_tables,
                        const int32_t* d_context_lens, const int32_t* table_rows, int n_seqs, int max_blocks_per_seq,
                        int num_q_heads, const resolved& r, void* d_workspace, hipStream_t st,
                        const call_events& ev) {
  const kv_pool_config& c = pool->cfg;
  const int64_t layer_off = static_cast<int64_t>(layer) * c.num_blocks * c.num_kv_heads * tile_bytes(c);
  const void* k_layer = static_cast<const char*>(pool->k_cache) + layer_off;
  const void* v_layer = static_cast<const char*>(pool->v_cache) + layer_off;
  const int G = num_q_heads / c.num_kv_heads;
  hipError_t e = hipSuccess;

  if (r.kernel == KV_KERNEL_MFMA) {
    sk_args a{};
    a.q = q;
    a.out = out;
    a.k_layer = k_layer;
    a.v_layer = v_layer;
    const uint64_t slots = static_cast<uint64_t>(r.groups) * kSkWaves + static_cast<uint64_t>(n_seqs) * c.num_kv_heads;
    char* ws = static_cast<char*>(d_workspace);
    a.part_m = reinterpret_cast<float*>(ws);
    a.part_l = reinterpret_cast<float*>(ws + up256(slots * G * 4));
    a.part_o = reinterpret_cast<float*>(ws + 2 * up256(slots * G * 4));
    a.cum_parts = reinterpret_cast<int32_t*>(ws + 2 * up256(slots * G * 4) + up256(slots * G * c.head_dim * 4));
    a.n_seqs = n_seqs;
    a.max_blocks = max_blocks_per_seq;
    a.n_q_heads = num_q_heads;
    a.n_kv_heads = c.num_kv_heads;
    a.num_blocks = c.num_blocks;
    a.part_blocks = r.partition / 16;  // partitions are whole 16-token tiles
    a.block_size = c.block_size;
    a.table_rows = table_rows;
    a.n_waves = static_cast<int>(r.groups * kSkWaves);
    a.q_units = sk_q_units(n_seqs, G, c.head_dim);
    a.scale_log2 = r.scale * kLog2e;
    auto launch = [&](auto fmt, auto bs) {
      constexpr int F = decltype(fmt)::value;
      constexpr int BS = decltype(bs)::value;
      switch (c.head_dim) {
        case 64: return launch_mfma<64, F, BS>(a, d_context_lens, d_block_tables, r.groups, G, st, ev.start, ev.kernel_stop, r.staged_table, r.valu);
        case 128: return launch_mfma<128, F, BS>(a, d_context_lens, d_block_tables, r.groups, G, st, ev.start, ev.kernel_stop, r.staged_table, r.valu);
        default: return launch_mfma<256, F, BS>(a, d_context_lens, d_block_tables, r.groups, G, st, ev.start, ev.kernel_stop, r.staged_table, r.valu);
      }
    };
    using B16 = std::integral_constant<int, 16>;
    if (c.dtype == KV_Q8_0) e = launch(std::integral_constant<int, kFmtQ8>{}, B16{});
    else if (c.dtype == KV_Q4_0) e = launch(std::integral_constant<int, kFmtQ4>{}, B16{});
    else {
      using BF = std::integral_constant<int, kFmtBf16>;
      switch (c.block_size) {
        case 4: e = launch(BF{}, std::integral_constant<int, 4>{}); break;
        case 8: e = launch(BF{}, std::integral_constant<int, 8>{}); break;
        case 32: e = launch(BF{}, std::integral_constant<int, 32>{}); break;
        case 64: e = launch(BF{}, std::integral_constant<int, 64>{}); break;
        default: e = launch(BF{}, B16{}); break;
      }
    }
    if (kv_status s = hip_check(e, "paged_attention_decode launch")) return s;
    const unsigned mgrid =
        static_cast<unsigned>((static_cast<int64_t>(n_seqs) * num_q_heads + kMergeItems - 1) / kMergeItems);
    switch (c.head_dim) {
      case 64: e = launch_timed(merge_sk_kernel<64>, dim3(mgrid), dim3(kMergeItems * 64), 0u, st, nullptr, ev.stop, a); break;
      case 128: e = launch_timed(merge_sk_kernel<128>, dim3(mgrid), dim3(kMergeItems * 64), 0u, st, nullptr, ev.stop, a); break;
      default: e = launch_timed(merge_sk_kernel<256>, dim3(mgrid), dim3(kMergeItems * 64), 0u, st, nullptr, ev.stop, a); break;
    }
    return hip_check(e, "paged attention merge launch");
  }

  const int64_t grid = static_cast<int64_t>(n_seqs) * c.num_kv_heads * r.max_parts;
  if (grid > 0x7fffffff) return fail(KV_ERR_INVALID, "grid too large");
  attn_args a{};
  a.q = q;
  a.out = out;
  a.tables = d_block_tables;
  a.ctx_lens = d_context_lens;
  a.k_layer = k_layer;
  a.v_layer = v_layer;
  if (r.max_parts > 1) {  // the partials need the workspace (workspace_for)
    const uint64_t rows = static_cast<uint64_t>(n_seqs) * num_q_heads * r.max_parts;
    char* ws = static_cast<char*>(d_workspace);
    a.part_m = reinterpret_cast<float*>(ws);
    a.part_l = reinterpret_cast<float*>(ws + up256(rows * 4));
    a.part_o = reinterpret_cast<float*>(ws + 2 * up256(rows * 4));
  }
  a.n_seqs = n_seqs;
  a.max_blocks = max_blocks_per_seq;
  a.n_q_heads = num_q_heads;
  a.n_kv_heads = c.num_kv_heads;
  a.head_dim = c.head_dim;
  a.block_size = c.block_size;
  a.num_blocks = c.num_blocks;
  a.partition_tokens = r.partition;
  a.max_parts = r.max_parts;
  a.scale_log2 = r.scale * kLog2e;
  a.table_rows = table_rows;
  const bool f32 = c.dtype == KV_F32;
  auto gen = [&](auto d) {
    constexpr int Dv = decltype(d)::value;
    return f32 ? launch_generic<float, Dv>(a, grid, st, ev.start, ev.kernel_stop)
               : launch_generic<uint16_t, Dv>(a, grid, st, ev.start, ev.kernel_stop);
  };
  switch (c.head_dim) {
    case 32: e = gen(std::integral_constant<int, 32>{}); break;
    case 64: e = gen(std::integral_constant<int, 64>{}); break;
    case 96: e = gen(std::integral_constant<int, 96>{}); break;
    case 128: e = gen(std::integral_constant<int, 128>{}); break;
    case 160: e = gen(std::integral_constant<int, 160>{}); break;
    case 192: e = gen(std::integral_constant<int, 192>{}); break;
    case 224: e = gen(std::integral_constant<int, 224>{}); break;
    default: e = gen(std::integral_constant<int, 256>{}); break;
  }
  if (kv_status s = hip_check(e, "paged_attention_decode launch")) return s;
  if (r.max_parts > 1) {
    const dim3 mgrid(static_cast<unsigned>(static_cast<int64_t>(n_seqs) * num_q_heads));
    e = f32 ? launch_timed(merge_kernel<float>, mgrid, dim3(kMergeThreads), 0u, st, nullptr, ev.stop, a)
            : launch_timed(merge_kernel<uint16_t>, mgrid, dim3(kMergeThreads), 0u, st, nullptr, ev.stop, a);
    return hip_check(e, "paged attention merge launch");
  }
  if (ev.stop) return hip_check(hipEventRecord(ev.stop, st), "timing event");
  return KV_OK;
}


// Row-wise multi-query path: rows go to the decode kernels in batches (the
// split-K kernel takes at most kSkMaxSeqs sequences per launch).  Workspace:
// per-row lengths and table rows, then the decode workspace of one batch.
struct rowwise_plan {
  resolved r;
  int batch;
  uint64_t rows_bytes, decode_off, total;
};

kv_status plan_rowwise(const kv_pool* pool, int total_q, int num_q_heads, int max_blocks,
                       const kv_attention_options* opts, rowwise_plan& p) {
  const int first = std::max(1, std::min(total_q, kSkMaxSeqs));
  if (kv_status s = resolve(pool, first, num_q_heads, max_blocks, opts, p.r)) return s;
  p.batch = p.r.kernel == KV_KERNEL_MFMA ? first : std::max(total_q, 1);
  if (p.batch != first)  // the generic kernel takes every row at once; its partition depends on the count
    if (kv_status s = resolve(pool, p.batch, num_q_heads, max_blocks, opts, p.r)) return s;
  p.rows_bytes = up256(static_cast<uint64_t>(std::max(total_q, 1)) * 4);
  p.decode_off = 2 * p.rows_bytes;
  p.total = p.decode_off + up256(workspace_for(pool->cfg, p.batch, num_q_heads, p.r));
  return KV_OK;
}

}  // namespace

uint64_t prefill_rowwise_workspace(const kv_pool* pool, int total_q, int num_q_heads, int max_blocks,
                                   const kv_attention_options* opts) {
  rowwise_plan p;
  if (plan_rowwise(pool, total_q, num_q_heads, max_blocks, opts, p) != KV_OK) return 0;
  return p.total;
}

kv_status prefill_rowwise(kv_pool* pool, int layer, const void* q, void* out, const int32_t* q_indptr,
                          const int32_t* tables, const int32_t* ctx, int n_seqs, int total_q, int max_q_len,
                          int max_blocks, int num_q_heads, const kv_attention_options* opts, void* ws,
                          uint64_t ws_bytes, hipStream_t st) {
  const kv_pool_config& c = pool->cfg;
  rowwise_plan p;
  if (kv_status s = plan_rowwise(pool, total_q, num_q_heads, max_blocks, opts, p)) return s;
  if (!ws || ws_bytes < p.total)
    return fail(KV_ERR_INVALID, "workspace too small: need " + std::to_string(p.total) + " bytes");
  if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(KV_ERR_INVALID, "workspace must be 256-byte aligned");
  const call_events ev = events_of(opts);
  char* w = static_cast<char*>(ws);
  int32_t* row_len = reinterpret_cast<int32_t*>(w);
  int32_t* row_table = reinterpret_cast<int32_t*>(w + p.rows_bytes);
  const unsigned grid = static_cast<unsigned>((total_q + 255) / 256);
  if (kv_status s = hip_check(launch_timed(prefill_rows_kernel, dim3(grid), dim3(256), 0u, st, ev.start, nullptr,
                                           q_indptr, ctx, n_seqs, total_q, max_q_len, max_blocks * c.block_size,
                                           row_len, row_table),
                              "prefill row lengths launch"))
    return s;
  // q and out rows in the pool's element type (bf16 for quantised pools)
  const int64_t row_bytes = static_cast<int64_t>(num_q_heads) * c.head_dim * (c.dtype == KV_F32 ? 4 : 2);
  for (int b0 = 0; b0 < total_q; b0 += p.batch) {
    const int n = std::min(p.batch, total_q - b0);
    const bool last = b0 + p.batch >= total_q;
    call_events e;
    e.kernel_stop = last ? ev.kernel_stop : nullptr;
    e.stop = last ? ev.stop : nullptr;
    if (kv_status s = decode_launch(pool, layer, static_cast<const char*>(q) + b0 * row_bytes,
                                    static_cast<char*>(out) + b0 * row_bytes, tables, row_len + b0, row_table + b0,
                                    n, max_blocks, num_q_heads, p.r, w + p.decode_off, st, e))
      return s;
  }
  return KV_OK;
}

}  // namespace pagedkv

using namespace pagedkv;

// ---- allocation-free decode -------------------------------------------------
// Scratch of paged_attention_decode_static: what paged_attention_decode takes as
// its caller's workspace (the split-K partials m, l, O of the runs that end
// inside a (sequence, kv head) unit, and the partition prefix), in one static
// device array that every GPU holds, at its own address, until the process
// ends.  Host code never passes the array's name to a kernel (on the host it
// stands for a host-side shadow, not device memory): the device address is
// looked up once per device with hipGetSymbolAddress and kept per device.
// Nothing in it needs to start at zero -- every partial a merge reads was
// written by the same call -- so it is never cleared.
static constexpr uint64_t kDecodeScratchBytes = 32ull << 20;
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call on that device).
kv_status decode_scratch(void** out) {
  int dev = -1;
  if (kv_status s = hip_check(hipGetDevice(&dev), "hipGetDevice")) return s;
  if (dev < 0 || dev >= kScratchDevices) return fail(KV_ERR_UNSUPPORTED, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (kv_status s = hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"))
      return s;
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255)) return fail(KV_ERR_HIP, "scratch address is not 256-byte aligned");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KV_OK;
}

}  // namespace

extern "C" {

uint64_t paged_attention_static_scratch_bytes(void) { return kDecodeScratchBytes; }

kv_status reshape_and_cache(kv_pool* pool, int32_t layer, const void* k_new, const void* v_new,
                            const int64_t* d_slot_mapping, int32_t n_tokens, void* hip_stream) {
  if (!pool) return fail(KV_ERR_INVALID, "pool is NULL");
  const kv_pool_config& c = pool->cfg;
  if (layer < 0 || layer >= c.num_layers) return fail(KV_ERR_INVALID, "layer out of range");
  if (n_tokens < 0) return fail(KV_ERR_INVALID, "n_tokens < 0");
  if (n_tokens == 0) return KV_OK;
  if (!k_new || !v_new || !d_slot_mapping || !pool->k_cache || !pool->v_cache)
    return fail(KV_ERR_INVALID, "NULL device pointer");
  if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) & 15)
    return fail(KV_ERR_INVALID, "k_new and v_new must be 16-byte aligned");
  if (is_quantized(c.dtype)) {
    const int64_t layer_bytes = static_cast<int64_t>(layer) * c.num_blocks * c.num_kv_heads * tile_bytes(c);
    unsigned char* kl = static_cast<unsigned char*>(pool->k_cache) + layer_bytes;
    unsigned char* vl = static_cast<unsigned char*>(pool->v_cache) + layer_bytes;
    const int64_t items = static_cast<int64_t>(n_tokens) * c.num_kv_heads * (c.head_dim / 32);
    const int64_t want = (items + 255) / 256;
    const unsigned grid = static_cast<unsigned>(want < 65536 ? want : 65536);
    const int64_t n_slots = static_cast<int64_t>(c.num_blocks) * c.block_size;
    const uint16_t* kn = static_cast<const uint16_t*>(k_new);
    const uint16_t* vn = static_cast<const uint16_t*>(v_new);
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    auto go = [&](auto d, auto f) {
      constexpr int D = decltype(d)::value, F = decltype(f)::value;
      hipLaunchKernelGGL((quantize_cache_kernel<D, F>), dim3(grid), dim3(256), 0, st, kn, vn, d_slot_mapping, kl, vl,
                         items, c.num_kv_heads, n_slots);
    };
    auto go_d = [&](auto f) {
      switch (c.head_dim) {
        case 64: go(std::integral_constant<int, 64>{}, f); break;
        case 128: go(std::integral_constant<int, 128>{}, f); break;
        default: go(std::integral_constant<int, 256>{}, f); break;
      }
    };
    if (c.dtype == KV_Q8_0) go_d(std::integral_constant<int, kFmtQ8>{});
    else go_d(std::integral_constant<int, kFmtQ4>{});
    return hip_check(hipGetLastError(), "reshape_and_cache launch");
  }
  const int64_t layer_off = static_cast<int64_t>(layer) * c.num_blocks * c.num_kv_heads * tile_elems(c);
  const int64_t n_slots = static_cast<int64_t>(c.num_blocks) * c.block_size;
  const int X = 16 / elem_bytes(c.dtype);
  const int64_t items = static_cast<int64_t>(n_tokens) * c.num_kv_heads * (c.head_dim / X);
  const int64_t want = (items + 255) / 256;
  const unsigned grid = static_cast<unsigned>(want < 65536 ? want : 65536);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (c.dtype == KV_F32) {
    hipLaunchKernelGGL(reshape_and_cache_kernel<float>, dim3(grid), dim3(256), 0, st, static_cast<const float*>(k_new),
                       static_cast<const float*>(v_new), d_slot_mapping, static_cast<float*>(pool->k_cache) + layer_off,
                       static_cast<float*>(pool->v_cache) + layer_off, items, c.num_kv_heads, c.head_dim, c.block_size,
                       n_slots);
  } else {
    hipLaunchKernelGGL(reshape_and_cache_kernel<uint16_t>, dim3(grid), dim3(256), 0, st,
                       static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), d_slot_mapping,
                       static_cast<uint16_t*>(pool->k_cache) + layer_off,
                       static_cast<uint16_t*>(pool->v_cache) + layer_off, items, c.num_kv_heads, c.head_dim,
                       c.block_size, n_slots);
  }
  if (kv_status s = hip_check(hipGetLastError(), "reshape_and_cache launch")) return s;
  return KV_OK;
}

kv_status copy_blocks(kv_pool* pool, const int64_t* d_pairs, int32_t n_pairs, void* hip_stream) {
  if (!pool) return fail(KV_ERR_INVALID, "pool is NULL");
  if (n_pairs < 0) return fail(KV_ERR_INVALID, "n_pairs < 0");
  if (n_pairs == 0) return KV_OK;
  if (!d_pairs || !pool->k_cache || !pool->v_cache) return fail(KV_ERR_INVALID, "NULL device pointer");
  const kv_pool_config& c = pool->cfg;
  const int64_t grid = static_cast<int64_t>(n_pairs) * c.num_layers * 2;
  if (grid > 0x7fffffff) return fail(KV_ERR_INVALID, "too many pairs");
  const int64_t block_bytes = static_cast<int64_t>(c.num_kv_heads) * tile_bytes(c);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                     static_cast<hipStream_t>(hip_stream), static_cast<uint4*>(pool->k_cache),
                     static_cast<uint4*>(pool->v_cache), d_pairs, c.num_layers, c.num_blocks, block_bytes / 16);
  return hip_check(hipGetLastError(), "copy_blocks launch");
}

uint64_t paged_attention_workspace_bytes(const kv_pool* pool, int32_t n_seqs, int32_t num_q_heads,
                                         int32_t max_blocks_per_seq, const kv_attention_options* opts) {
  if (!pool) return 0;
  resolved r;
  if (resolve(pool, n_seqs, num_q_heads, max_blocks_per_seq, opts, r) != KV_OK) return 0;
  return workspace_for(pool->cfg, n_seqs, num_q_heads, r);
}

kv_status paged_attention_decode(kv_pool* pool, int32_t layer, const void* q, void* out,
                                 const int32_t* d_block_tables, const int32_t* d_context_lens, int32_t n_seqs,
                                 int32_t max_blocks_per_seq, int32_t num_q_heads, const kv_attention_options* opts,
                                 void* d_workspace, uint64_t workspace_bytes, void* hip_stream) {
  if (!pool) return fail(KV_ERR_INVALID, "pool is NULL");
  const kv_pool_config& c = pool->cfg;
  if (layer < 0 || layer >= c.num_layers) return fail(KV_ERR_INVALID, "layer out of range");
  resolved r;
  if (kv_status s = resolve(pool, n_seqs, num_q_heads, max_blocks_per_seq, opts, r)) return s;
  if (n_seqs == 0) return KV_OK;
  if (!q || !out || !d_block_tables || !d_context_lens || !pool->k_cache || !pool->v_cache)
    return fail(KV_ERR_INVALID, "NULL device pointer");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out)) & 15)
    return fail(KV_ERR_INVALID, "q and out must be 16-byte aligned");
  const uint64_t need = workspace_for(c, n_seqs, num_q_heads, r);
  if (need > 0 && (!d_workspace || workspace_bytes < need))
    return fail(KV_ERR_INVALID, "workspace too small: need " + std::to_string(need) + " bytes");
  if (need > 0 && (reinterpret_cast<uintptr_t>(d_workspace) & 255))
    return fail(KV_ERR_INVALID, "workspace must be 256-byte aligned");
  const hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const call_events ev = events_of(opts);
  if (r.kernel != KV_KERNEL_MFMA || n_seqs <= kSkMaxSeqs)
    return decode_launch(pool, layer, q, out, d_block_tables, d_context_lens, nullptr, n_seqs, max_blocks_per_seq,
                         num_q_heads, r, d_workspace, st, ev);
  // more sequences than one launch takes: consecutive launches over slices of
  // the batch, reusing the workspace (stream order separates them); the timing
  // events go to the first launch's start and the last launch's ends
  const int64_t row_bytes = static_cast<int64_t>(num_q_heads) * c.head_dim * 2;  // bf16 q / out rows
  for (int b0 = 0; b0 < n_seqs; b0 += kSkMaxSeqs) {
    const int n = std::min(kSkMaxSeqs, n_seqs - b0);
    const bool last = b0 + kSkMaxSeqs >= n_seqs;
    call_events e;
    e.start = b0 == 0 ? ev.start : nullptr;
    e.kernel_stop = last ? ev.kernel_stop : nullptr;
    e.stop = last ? ev.stop : nullptr;
    if (kv_status s = decode_launch(pool, layer, static_cast<const char*>(q) + b0 * row_bytes,
                                    static_cast<char*>(out) + b0 * row_bytes,
                                    d_block_tables + static_cast<int64_t>(b0) * max_blocks_per_seq,
                                    d_context_lens + b0, nullptr, n, max_blocks_per_seq, num_q_heads, r, d_workspace,
                                    st, e))
      return s;
  }
  return KV_OK;
}

kv_status paged_attention_decode_static(kv_pool* pool, int32_t layer, const void* q, void* out,
                                        const int32_t* d_block_tables, const int32_t* d_context_lens, int32_t n_seqs,
                                        int32_t max_blocks_per_seq, int32_t num_q_heads,
                                        const kv_attention_options* opts, void* hip_stream) {
  if (!pool) return fail(KV_ERR_INVALID, "pool is NULL");
  resolved r;
  if (kv_status s = resolve(pool, n_seqs, num_q_heads, max_blocks_per_seq, opts, r)) return s;
  const uint64_t need = workspace_for(pool->cfg, n_seqs, num_q_heads, r);
  if (need > kDecodeScratchBytes)
    return fail(KV_ERR_INVALID, "the call needs " + std::to_string(need) + " bytes of scratch, more than the " +
                                    std::to_string(kDecodeScratchBytes) +
                                    " of the static scratch; use paged_attention_decode with a workspace");
  void* ws = nullptr;
  if (need > 0)
    if (kv_status s = decode_scratch(&ws)) return s;
  return paged_attention_decode(pool, layer, q, out, d_block_tables, d_context_lens, n_seqs, max_blocks_per_seq,
                                num_q_heads, opts, ws, need > 0 ? kDecodeScratchBytes : 0, hip_stream);
}

}  // extern "C"
