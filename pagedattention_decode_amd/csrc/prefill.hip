// Multi-query attention over paged history for gfx950 (MI355X): chunked
// prefill and verification of draft positions.
//
// Sources (by page title):
//   [KVM] "KV 缓存管理": chunked prefill mechanism and Figure 8 — the queries of
//         chunk k attend the cached K/V of chunks 1..k-1 (all visible) and the
//         chunk's own tokens under a lower-triangular causal mask, with the
//         running maximum m, sum l and output O folded across blocks.
//   [INF] "第 8 章 推理优化": §8.2.3 — a chunk of c tokens over h cached tokens
//         forms c h + c(c+1)/2 query-key pairs; §8.5.1 — the target model scores
//         all draft positions of a request in one pass.
//
// The chunk's own K/V rows are in the pool before the call (reshape_and_cache),
// so sequence s holds n = context_lens[s] tokens, its c queries are the last c
// positions h = n - c .. n - 1, and the query at chunk row j sees positions
// 0 .. h + j.
//
// Work split.  Unit = (sequence, kv head).  Its queries are flattened into
// columns f = j * G + hg (chunk row j, query head g * G + hg).  A wave owns a
// tile of NC = 16 * NCG consecutive columns and one partition of the keys; the
// four waves of a workgroup own four consecutive tiles of one unit and the same
// partition, so they stream the same K/V blocks (the second to fourth reads hit
// in L2).  Per 16-token block and 16-column group, as in the decode kernel:
//   S^T[16 tokens][16 cols] = K[16][D] . Q^T[D][16]   (D/32 x mfma 16x16x32)
//   causal mask, online softmax (each lane holds 4 tokens of one column)
//   O^T[D][16 cols] += V^T[D][16] . P^T[16][16]        (D/16 x mfma 16x16x16)
// The block is loaded once for all NCG groups; a group skips the blocks past
// its last visible position.  A tile whose keys fit one partition writes its
// final rows; otherwise every partition writes (m, l, O) and merge_prefill
// folds them with the running-max recurrences.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <string>

#include "device_common.h"
#include "pool_internal.h"

namespace pagedkv {
namespace {

constexpr int kPfWaves = 4;  // waves (tiles) per workgroup

struct pf_args {
  const void* q;        // [total_q][Hq][D] bf16
  void* out;            // [total_q][Hq][D] bf16
  const void* k_layer;  // K pool of the layer
  const void* v_layer;  // V pool of the layer
  const int32_t* q_indptr;  // [n_seqs + 1]
  const int32_t* ctx_lens;  // [n_seqs]
  const int32_t* tables;    // [n_seqs][max_blocks]
  float* part_m;            // [total_q * Hq][max_parts]
  float* part_l;            // [total_q * Hq][max_parts]
  float* part_o;            // [total_q * Hq][max_parts][D]
  int n_seqs, total_q, max_q_len, max_blocks, n_q_heads, n_kv_heads, num_blocks;
  int part_blocks, max_parts, tile_groups, cols_per_tile;
  float scale_log2;
};

// One 16-token block for one 16-column group: scores, causal mask, online
// softmax, weighted values.  `lim` (per lane) is the number of leading slots
// of the block visible to this lane's column (0 .. 16).  The V tail beyond the
// context has already been zeroed.
template <int D>
__device__ __forceinline__ void attend_cols(const kv_regs<D>& cur, const bf16x8_t* qop, int lim, int quad,
                                            float scale_log2, f32x4_t* o, float& m_run, float& l_lane) {
  f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk)
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, cur.k[kk]), qop[kk], s, 0, 0, 0);

  float sv[4];
  float mb = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sv[i] = (quad * 4 + i < lim) ? s[i] * scale_log2 : -INFINITY;
    mb = fmaxf(mb, sv[i]);
  }
  mb = fmaxf(mb, __shfl_xor(mb, 16));
  mb = fmaxf(mb, __shfl_xor(mb, 32));
  const bool grow = mb > m_run + kRescaleSlack;
  if (__builtin_amdgcn_ballot_w64(grow)) {  // wave-uniform branch
    const float m_new = grow ? mb : m_run;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 when m_run = -inf, 1 when kept
    l_lane *= alpha;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) o[i] *= alpha;
    m_run = m_new;
  }
  float pv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pv[i] = (sv[i] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sv[i] - m_run);
  // P^T in bf16 (round to nearest even); the denominator sums the rounded
  // weights, so the weights applied to V are exactly normalised
  const bf16x2_t p01 = __builtin_convertvector((f32x2_t{pv[0], pv[1]}), bf16x2_t);
  const bf16x2_t p23 = __builtin_convertvector((f32x2_t{pv[2], pv[3]}), bf16x2_t);
  const uint32_t w01 = __builtin_bit_cast(uint32_t, p01);
  const uint32_t w23 = __builtin_bit_cast(uint32_t, p23);
  l_lane += (__uint_as_float(w01 << 16) + __uint_as_float(w01 & 0xffff0000u)) +
            (__uint_as_float(w23 << 16) + __uint_as_float(w23 & 0xffff0000u));
  const s16x4_t pop = __builtin_bit_cast(s16x4_t, make_uint2(w01, w23));
#pragma unroll
  for (int pp = 0; pp < D / 32; ++pp) {
    const uint2* halves = reinterpret_cast<const uint2*>(&cur.v[pp]);
    o[2 * pp] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, halves[0]), pop, o[2 * pp],
                                                          0, 0, 0);
    o[2 * pp + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, halves[1]), pop,
                                                              o[2 * pp + 1], 0, 0, 0);
  }
}

// Where a sequence's queries are and whether its arguments are usable.
struct pf_seq {
  int q0, c, n, h;  // first query row, chunk length, context, history
  bool bad;         // chunk longer than the context or than max_q_len: NaN rows
};

__device__ __forceinline__ pf_seq pf_locate(const pf_args& a, int s) {
  pf_seq r;
  r.q0 = a.q_indptr[s];
  r.c = a.q_indptr[s + 1] - r.q0;
  r.n = min(a.ctx_lens[s], a.max_blocks * 16);
  r.h = r.n - r.c;
  r.bad = r.c > a.max_q_len || r.c > r.n;
  return r;
}

// Keys [0, kend) of tile `tile` of a sequence: up to the position of its last column.
__device__ __forceinline__ int pf_tile_keys(const pf_seq& q, int G, int tile, int nc) {
  const int f_last = min((tile + 1) * nc, q.c * G) - 1;
  return q.h + f_last / G + 1;
}

template <int D, int NCG>
__global__ void __launch_bounds__(kPfWaves * 64) attn_prefill_kernel(pf_args a) {
  constexpr int NC = 16 * NCG;
  const int lane = threadIdx.x & 63;
  const int quad = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int bid = blockIdx.x;
  const int part = bid % a.max_parts;
  bid /= a.max_parts;
  const int tg = bid % a.tile_groups;
  bid /= a.tile_groups;
  const int g = bid % a.n_kv_heads;
  const int s = bid / a.n_kv_heads;
  const int G = a.n_q_heads / a.n_kv_heads;
  const int tile = tg * kPfWaves + wave;

  const pf_seq sq = pf_locate(a, s);
  if (sq.c <= 0 || sq.q0 < 0 || sq.q0 + sq.c > a.total_q) return;  // nothing, or rows outside the output
  const int cols = sq.c * G;
  uint16_t* out = static_cast<uint16_t*>(a.out);
  if (sq.bad) {  // one wave per unit marks the unit's rows
    if (part == 0 && tile == 0)
      for (int i = lane; i < cols * D; i += 64) {
        const int f = i / D, e = i % D;
        out[(static_cast<int64_t>(sq.q0 + f / G) * a.n_q_heads + g * G + f % G) * D + e] = 0x7fc0;
      }
    return;
  }
  if (tile * NC >= cols) return;
  const int kend = pf_tile_keys(sq, G, tile, NC);
  const int P = a.part_blocks * 16;
  const int k_begin = part * P;
  if (k_begin >= kend) return;
  const int n_parts = (kend + P - 1) / P;
  const int b_begin = k_begin >> 4;
  const int b_end = (min(kend, k_begin + P) + 15) >> 4;
  const int f0 = tile * NC;

  // this lane's column in every group, and each group's last visible position
  bf16x8_t qop[NCG][D / 32];
  int pos[NCG];
  int gmax[NCG];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const int f = f0 + cg * 16 + (lane & 15);
    const bool live = f < cols;
    const int j = live ? f / G : 0;
    const int hg = live ? f % G : 0;
    pos[cg] = live ? sq.h + j : -1;
    gmax[cg] = (f0 + cg * 16 < cols) ? sq.h + min(f0 + cg * 16 + 15, cols - 1) / G : -1;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         (static_cast<int64_t>(sq.q0 + j) * a.n_q_heads + g * G + hg) * D + quad * 8;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
      qop[cg][kk] = live ? *reinterpret_cast<const bf16x8_t*>(qp + kk * 32) : bf16x8_t{};
  }

  const uint4* kpool = static_cast<const uint4*>(a.k_layer);
  const uint4* vpool = static_cast<const uint4*>(a.v_layer);
  constexpr int kTileVec = 16 * D * 2 / 16;  // 16-byte vectors per tile
  const int32_t* trow = a.tables + static_cast<int64_t>(s) * a.max_blocks;
  // two-deep register ring; loads past the run repeat its last block (L2 hits)
  kv_regs<D> buf[2];
  int phys_ring[2];
  auto issue = [&](int u, int b) {
    const int phys = trow[min(b, b_end - 1)];
    phys_ring[u] = phys;
    const int p = (phys < 0 || phys >= a.num_blocks) ? 0 : phys;  // never dereferenced out of range
    const int64_t t = (static_cast<int64_t>(p) * a.n_kv_heads + g) * kTileVec;
    load_block<D>(buf[u], kpool + t, vpool + t, lane);
  };

  f32x4_t o[NCG][D / 16];
  float m_run[NCG], l_lane[NCG];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
#pragma unroll
    for (int i = 0; i < D / 16; ++i) o[cg][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m_run[cg] = -INFINITY;
    l_lane[cg] = 0.f;
  }
  bool poisoned = false;

  issue(0, b_begin);
  issue(1, b_begin + 1);
  for (int b0 = b_begin; b0 < b_end; b0 += 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int b = b0 + u;
      if (b < b_end) {
        const int phys = phys_ring[u];
        const bool bad = phys < 0 || phys >= a.num_blocks;
        poisoned |= bad;
        const int valid = bad ? 0 : min(16, sq.n - b * 16);
        if (valid < 16) zero_v_tail<D>(buf[u], valid, quad);
#pragma unroll
        for (int cg = 0; cg < NCG; ++cg) {
          if (b * 16 > gmax[cg]) continue;  // wave-uniform: the whole group is masked
          const int lim = min(max(min(pos[cg] - b * 16 + 1, valid), 0), 16);
          attend_cols<D>(buf[u], qop[cg], lim, quad, a.scale_log2, o[cg], m_run[cg], l_lane[cg]);
        }
      }
      issue(u, b + 2);
    }
  }

  const float nan = __builtin_nanf("");
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    float l = l_lane[cg] + __shfl_xor(l_lane[cg], 16);
    l += __shfl_xor(l, 32);
    const int f = f0 + cg * 16 + (lane & 15);
    if (f >= cols) continue;
    const int64_t row = static_cast<int64_t>(sq.q0 + f / G) * a.n_q_heads + g * G + f % G;
    if (n_parts == 1) {
      const float inv = 1.f / l;
      uint16_t* orow = out + row * D;
#pragma unroll
      for (int nt = 0; nt < D / 16; ++nt) {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = poisoned ? nan : o[cg][nt][i] * inv;
        *reinterpret_cast<uint2*>(orow + nt * 16 + quad * 4) =
            make_uint2(static_cast<uint32_t>(f32_to_bf16(v[0])) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16),
                       static_cast<uint32_t>(f32_to_bf16(v[2])) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16));
      }
    } else {
      const int64_t pi = row * a.max_parts + part;
      float* po = a.part_o + pi * D;
#pragma unroll
      for (int nt = 0; nt < D / 16; ++nt)
        *reinterpret_cast<float4*>(po + nt * 16 + quad * 4) =
            poisoned ? make_float4(nan, nan, nan, nan)
                     : make_float4(o[cg][nt][0], o[cg][nt][1], o[cg][nt][2], o[cg][nt][3]);
      if (quad == 0) {
        a.part_m[pi] = poisoned ? nan : m_run[cg];
        a.part_l[pi] = poisoned ? nan : l;
      }
    }
  }
}

// Folds the partitions of every (query row, head) whose tile had more than one:
// M = max_p m_p, out = sum_p 2^(m_p - M) O_p / sum_p 2^(m_p - M) l_p.  A
// partition that saw no key of the row has m = -inf and weight 0; a poisoned
// one carries NaN into the row.  One wave per (row, head).
constexpr int kPfMergeWaves = 4;

template <int D>
__global__ void __launch_bounds__(kPfMergeWaves * 64) merge_prefill_kernel(pf_args a) {
  const int lane = threadIdx.x & 63;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * kPfMergeWaves + (threadIdx.x >> 6);
  if (item >= static_cast<int64_t>(a.total_q) * a.n_q_heads) return;
  const int r = static_cast<int>(item / a.n_q_heads);
  const int head = static_cast<int>(item % a.n_q_heads);
  // sequence of row r: the last s with q_indptr[s] <= r
  int lo = 0, hi = a.n_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.q_indptr[mid] <= r) lo = mid; else hi = mid - 1;
  }
  const pf_seq sq = pf_locate(a, lo);
  if (sq.c <= 0 || r < sq.q0 || r >= sq.q0 + sq.c || sq.bad) return;
  const int G = a.n_q_heads / a.n_kv_heads;
  const int f = (r - sq.q0) * G + head % G;
  const int kend = pf_tile_keys(sq, G, f / a.cols_per_tile, a.cols_per_tile);
  const int P = a.part_blocks * 16;
  const int n_parts = (kend + P - 1) / P;
  if (n_parts <= 1) return;
  const int64_t base = item * a.max_parts;
  float M = -INFINITY;
  bool nan_seen = false;
  for (int p = 0; p < n_parts; ++p) {
    const float m = a.part_m[base + p];
    nan_seen |= m != m;
    M = fmaxf(M, m);
  }
  constexpr int E = (D + 63) / 64;  // dims per lane
  float acc[E];
#pragma unroll
  for (int i = 0; i < E; ++i) acc[i] = 0.f;
  float L = 0.f;
  for (int p = 0; p < n_parts; ++p) {
    const float m = a.part_m[base + p];
    if (m == -INFINITY || m != m) continue;
    const float w = exp2f(m - M);
    L += w * a.part_l[base + p];
    const float* po = a.part_o + (base + p) * D;
#pragma unroll
    for (int i = 0; i < E; ++i)
      if (lane + 64 * i < D) acc[i] += w * po[lane + 64 * i];
  }
  uint16_t* orow = static_cast<uint16_t*>(a.out) + item * D;
#pragma unroll
  for (int i = 0; i < E; ++i)
    if (lane + 64 * i < D) orow[lane + 64 * i] = f32_to_bf16(nan_seen ? __builtin_nanf("") : acc[i] / L);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

struct pf_plan {
  int ncg;          // 16-column groups per wave
  int tiles;        // tiles per sequence (upper bound)
  int tile_groups;  // workgroups per (sequence, kv head, partition)
  int partition;    // tokens per partition
  int max_parts;
  float scale;
};

kv_status pf_resolve(const kv_pool* pool, int n_seqs, int total_q, int max_q_len, int num_q_heads, int max_blocks,
                     const kv_attention_options* opts, pf_plan& p) {
  if (!pool) return fail(KV_ERR_INVALID, "pool is NULL");
  const kv_pool_config& c = pool->cfg;
  if (num_q_heads <= 0 || num_q_heads % c.num_kv_heads != 0)
    return fail(KV_ERR_INVALID, "num_q_heads must be a positive multiple of num_kv_heads");
  const int G = num_q_heads / c.num_kv_heads;
  if (n_seqs < 0 || total_q < 0 || max_blocks <= 0 || max_q_len <= 0)
    return fail(KV_ERR_INVALID, "n_seqs, total_q >= 0 and max_q_len, max_blocks_per_seq > 0 required");
  kv_attention_options o{0.f, 0, KV_KERNEL_AUTO};
  if (opts) o = *opts;
  if (o.kernel != KV_KERNEL_AUTO && o.kernel != KV_KERNEL_MFMA)
    return fail(KV_ERR_UNSUPPORTED, "multi-query attention has only the matrix-core kernel");
  if (!mfma_supported(c, G))
    return fail(KV_ERR_UNSUPPORTED, "multi-query attention needs bf16, B = 16, d in {64, 128, 256} and G <= 16");
  if (o.partition_tokens < 0 || o.partition_tokens % 16 != 0)
    return fail(KV_ERR_INVALID, "partition_tokens must be 0 or a positive multiple of the block size");
  if (!(o.scale >= 0.f) || std::isinf(o.scale)) return fail(KV_ERR_INVALID, "scale must be finite and >= 0");
  p.scale = o.scale > 0.f ? o.scale : 1.f / std::sqrt(static_cast<float>(c.head_dim));
  const int64_t cols = static_cast<int64_t>(max_q_len) * G;
  const int max_ncg = c.head_dim >= 256 ? 2 : 4;
  p.ncg = cols <= 16 ? 1 : (cols <= 32 || max_ncg == 2 ? 2 : 4);
  p.tiles = static_cast<int>((cols + 16 * p.ncg - 1) / (16 * p.ncg));
  p.tile_groups = (p.tiles + kPfWaves - 1) / kPfWaves;
  const int64_t max_ctx = static_cast<int64_t>(max_blocks) * 16;
  if (o.partition_tokens > 0) {
    p.partition = o.partition_tokens;
  } else {
    // enough waves for two per SIMD; otherwise one partition per tile
    const int64_t waves = static_cast<int64_t>(n_seqs) * c.num_kv_heads * p.tiles;
    const int64_t want = 8LL * device_cus();
    if (waves >= want) {
      p.partition = static_cast<int>(max_ctx);
    } else {
      const int64_t parts = (want + std::max<int64_t>(waves, 1) - 1) / std::max<int64_t>(waves, 1);
      const int64_t per = ((max_ctx + parts - 1) / parts + 15) / 16 * 16;
      p.partition = static_cast<int>(std::max<int64_t>(256, per));
    }
  }
  p.max_parts = static_cast<int>((max_ctx + p.partition - 1) / p.partition);
  const int64_t grid = static_cast<int64_t>(n_seqs) * c.num_kv_heads * p.tile_groups * p.max_parts;
  if (grid > 0x7fffffff) return fail(KV_ERR_INVALID, "grid too large");
  return KV_OK;
}

uint64_t pf_workspace(const kv_pool_config& c, int total_q, int num_q_heads, const pf_plan& p) {
  if (p.max_parts <= 1) return 0;
  const uint64_t rows = static_cast<uint64_t>(total_q) * num_q_heads * p.max_parts;
  return 2 * up256(rows * 4) + up256(rows * c.head_dim * 4);
}

template <int D, int NCG>
hipError_t pf_launch(const pf_args& a, int64_t grid, hipStream_t st) {
  hipLaunchKernelGGL((attn_prefill_kernel<D, NCG>), dim3(static_cast<unsigned>(grid)), dim3(kPfWaves * 64), 0, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t pf_launch_d(const pf_args& a, int ncg, int64_t grid, hipStream_t st) {
  if (ncg == 1) return pf_launch<D, 1>(a, grid, st);
  if (ncg == 2) return pf_launch<D, 2>(a, grid, st);
  if constexpr (D < 256) return pf_launch<D, 4>(a, grid, st);
  return hipErrorInvalidValue;
}

template <int D>
hipError_t pf_merge(const pf_args& a, hipStream_t st) {
  const int64_t items = static_cast<int64_t>(a.total_q) * a.n_q_heads;
  const int64_t grid = (items + kPfMergeWaves - 1) / kPfMergeWaves;
  hipLaunchKernelGGL((merge_prefill_kernel<D>), dim3(static_cast<unsigned>(grid)), dim3(kPfMergeWaves * 64), 0, st,
                     a);
  return hipGetLastError();
}

}  // namespace
}  // namespace pagedkv

using namespace pagedkv;

extern "C" {

uint64_t paged_prefill_workspace_bytes(const kv_pool* pool, int32_t n_seqs, int32_t total_q, int32_t max_q_len,
                                       int32_t num_q_heads, int32_t max_blocks_per_seq,
                                       const kv_attention_options* opts) {
  pf_plan p;
  if (pf_resolve(pool, n_seqs, total_q, max_q_len, num_q_heads, max_blocks_per_seq, opts, p) != KV_OK) return 0;
  return pf_workspace(pool->cfg, total_q, num_q_heads, p);
}

kv_status paged_attention_prefill(kv_pool* pool, int32_t layer, const void* q, void* out, const int32_t* d_q_indptr,
                                  const int32_t* d_block_tables, const int32_t* d_context_lens, int32_t n_seqs,
                                  int32_t total_q, int32_t max_q_len, int32_t max_blocks_per_seq,
                                  int32_t num_q_heads, const kv_attention_options* opts, void* d_workspace,
                                  uint64_t workspace_bytes, void* hip_stream) {
  pf_plan p;
  if (kv_status s = pf_resolve(pool, n_seqs, total_q, max_q_len, num_q_heads, max_blocks_per_seq, opts, p)) return s;
  const kv_pool_config& c = pool->cfg;
  if (layer < 0 || layer >= c.num_layers) return fail(KV_ERR_INVALID, "layer out of range");
  if (n_seqs == 0 || total_q == 0) return KV_OK;
  if (!q || !out || !d_q_indptr || !d_block_tables || !d_context_lens || !pool->k_cache || !pool->v_cache)
    return fail(KV_ERR_INVALID, "NULL device pointer");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out)) & 15)
    return fail(KV_ERR_INVALID, "q and out must be 16-byte aligned");
  const uint64_t need = pf_workspace(c, total_q, num_q_heads, p);
  if (need > 0 && (!d_workspace || workspace_bytes < need))
    return fail(KV_ERR_INVALID, "workspace too small: need " + std::to_string(need) + " bytes");
  if (need > 0 && (reinterpret_cast<uintptr_t>(d_workspace) & 255))
    return fail(KV_ERR_INVALID, "workspace must be 256-byte aligned");
  const int64_t layer_off =
      static_cast<int64_t>(layer) * c.num_blocks * c.num_kv_heads * tile_elems(c) * elem_bytes(c.dtype);
  pf_args a{};
  a.q = q;
  a.out = out;
  a.k_layer = static_cast<const char*>(pool->k_cache) + layer_off;
  a.v_layer = static_cast<const char*>(pool->v_cache) + layer_off;
  a.q_indptr = d_q_indptr;
  a.ctx_lens = d_context_lens;
  a.tables = d_block_tables;
  if (need > 0) {
    const uint64_t rows = static_cast<uint64_t>(total_q) * num_q_heads * p.max_parts;
    char* ws = static_cast<char*>(d_workspace);
    a.part_m = reinterpret_cast<float*>(ws);
    a.part_l = reinterpret_cast<float*>(ws + up256(rows * 4));
    a.part_o = reinterpret_cast<float*>(ws + 2 * up256(rows * 4));
  }
  a.n_seqs = n_seqs;
  a.total_q = total_q;
  a.max_q_len = max_q_len;
  a.max_blocks = max_blocks_per_seq;
  a.n_q_heads = num_q_heads;
  a.n_kv_heads = c.num_kv_heads;
  a.num_blocks = c.num_blocks;
  a.part_blocks = p.partition / 16;
  a.max_parts = p.max_parts;
  a.tile_groups = p.tile_groups;
  a.cols_per_tile = 16 * p.ncg;
  a.scale_log2 = p.scale * kLog2e;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const int64_t grid = static_cast<int64_t>(n_seqs) * c.num_kv_heads * p.tile_groups * p.max_parts;
  hipError_t e;
  switch (c.head_dim) {
    case 64: e = pf_launch_d<64>(a, p.ncg, grid, st); break;
    case 128: e = pf_launch_d<128>(a, p.ncg, grid, st); break;
    default: e = pf_launch_d<256>(a, p.ncg, grid, st); break;
  }
  if (kv_status s = hip_check(e, "paged_attention_prefill launch")) return s;
  if (p.max_parts > 1) {
    switch (c.head_dim) {
      case 64: e = pf_merge<64>(a, st); break;
      case 128: e = pf_merge<128>(a, st); break;
      default: e = pf_merge<256>(a, st); break;
    }
    return hip_check(e, "paged_attention_prefill merge launch");
  }
  return KV_OK;
}

}  // extern "C"
