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
// tile of NC = 16 * NCG consecutive columns and one partition of the keys.  The
// four waves of a workgroup own wt consecutive tiles (4 when a unit has that
// many) times 4 / wt consecutive partitions of one unit; waves on the same
// partition stream the same K/V blocks, so all but the first read hit in L2.
// Per 16-token block and 16-column group, as in the decode kernel:
//   S^T[16 tokens][16 cols] = K[16][D] . Q^T[D][16]   (D/32 x mfma 16x16x32)
//   causal mask, online softmax (each lane holds 4 tokens of one column)
//   O^T[D][16 cols] += V^T[D][16] . P^T[16][16]        (D/16 x mfma 16x16x16)
// The block is loaded once for all NCG groups; a group skips the blocks past
// its last visible position.  A tile whose keys fit one partition writes its
// final rows; otherwise every partition writes (m, l, O) and merge_prefill
// folds them with the running-max recurrences.
// The kernels work in 16-token tiles whatever the pool's block size B (4 ..
// 64: a table entry holds B/16 tiles, or a tile gathers 16/B entries), and a
// quantised pool (q8_0 / q4_0, B = 16, d <= 128) has a kernel of its own that
// feeds the codes to the matrix instructions and applies the group scales in
// float32 ([INF] §8.4.2).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <string>

#include "device_common.h"
#include "pool_internal.h"

namespace pagedkv {
namespace {

constexpr int kPfWaves = 4;  // waves per workgroup: wt tiles x (4 / wt) partitions

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
  int part_blocks, max_parts, cols_per_tile;
  int block_size;                // B: tokens per table entry (the kernels work in 16-token tiles)
  int wt;                        // tiles per workgroup (1, 2 or 4); the other factor of 4 is partitions
  int tile_groups, part_groups;  // workgroups per unit along tiles and along partitions
  float scale_log2;
  // Launch options.  The prefill sets causal = 1 and leaves the other two
  // off; with causal = 0 every query would see all n keys, table_rows remaps
  // "sequence" s to table row table_rows[s], and force_partial makes every
  // tile write partials even when it has one partition.
  int causal;
  int force_partial;
  const int32_t* table_rows;  // nullptr: row s
};

// Two consecutive 16-token blocks in registers.  K as for the decode kernel
// (the A operands of S^T = K Q^T); V regrouped for mfma 16x16x32 over the 32
// tokens: v[t] holds, for d-tile t (16 dims), the lane's 4 tokens of the first
// block in dwords 0-1 and its 4 tokens of the second block in dwords 2-3, so
// that it is the A operand of O^T += V^T P^T as loaded (two 8-byte loads from
// the two blocks' V tiles, same cache lines as one 16-byte load each).
template <int D>
struct kv_pair {
  uint4 ka[D / 32];
  uint4 kb[D / 32];
  uint4 v[D / 16];
};

// The lane's pieces: K piece i of a tile at kta[i * STRIDE], V piece i at
// vta[i * STRIDE] (the pointers already hold the lane's offset; STRIDE = 4 B
// in 16-byte units for block size B, 64 for B = 16).
template <int D, int STRIDE>
__device__ __forceinline__ void load_pair(kv_pair<D>& r, const uint4* kta, const uint4* vta, const uint4* ktb,
                                          const uint4* vtb) {
#pragma unroll
  for (int i = 0; i < D / 32; ++i) r.ka[i] = kta[i * STRIDE];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) r.kb[i] = ktb[i * STRIDE];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    const uint2* va = reinterpret_cast<const uint2*>(vta + i * STRIDE);
    const uint2* vb = reinterpret_cast<const uint2*>(vtb + i * STRIDE);
    const uint2 a0 = va[0], a1 = va[1], b0 = vb[0], b1 = vb[1];
    r.v[2 * i] = make_uint4(a0.x, a0.y, b0.x, b0.y);
    r.v[2 * i + 1] = make_uint4(a1.x, a1.y, b1.x, b1.y);
  }
}

// Masks that keep the V values of slots < valid_a of the first block and
// < valid_b of the second in a V operand (dwords 0-1: the lane's 4 slots of
// the first block, 2-3: of the second); memory past the context may hold
// anything.
struct v_tail_mask {
  uint32_t a[2], b[2];
  __device__ __forceinline__ v_tail_mask(int valid_a, int valid_b, int quad) {
#pragma unroll
    for (int dw = 0; dw < 2; ++dw) {
      const int slot0 = quad * 4 + dw * 2;
      a[dw] = (slot0 < valid_a ? 0x0000ffffu : 0u) | (slot0 + 1 < valid_a ? 0xffff0000u : 0u);
      b[dw] = (slot0 < valid_b ? 0x0000ffffu : 0u) | (slot0 + 1 < valid_b ? 0xffff0000u : 0u);
    }
  }
  __device__ __forceinline__ uint4 apply(uint4 v) const {
    return make_uint4(v.x & a[0], v.y & a[1], v.z & b[0], v.w & b[1]);
  }
};

// Two consecutive 16-token blocks (32 tokens) for all NCG 16-column groups.
//   1. S^T of both blocks for every group: 2 * NCG independent chains of
//      D/32 x mfma 16x16x32; the Q^T operands come from LDS (the wave's own
//      copy, in operand order), which leaves the registers to the K/V ring
//      and the accumulators.
//   2. Online softmax per group over the 8 scores a lane holds (tokens
//      4q..4q+3 of each block, q = lane / 16, for column lane % 16); one vote
//      over the wave decides whether any group's running maximum moves.  The
//      scale is applied in the exponent: p = 2^(s * c - m).
//   3. O^T += V^T P^T with mfma 16x16x32 over the 32 tokens: contraction index
//      k = 8q + i is token 4q + i of the first block for i < 4 and token
//      4q + i - 4 of the second for i >= 4 (the order of kv_pair::v), so the B
//      operand is the two blocks' P^T operands side by side.
// masked (wave uniform): `lim_a`, `lim_b` (per lane and group) are the
// numbers of leading slots of each block visible to the lane's column;
// otherwise every slot of both blocks is visible to every column.  V tails
// beyond the context are already zero.  (One instance serves both cases, so
// that the accumulators live in one set of registers: with two, the compiler
// moved all of them from one set to the other after every pair.)
// The operands come from callbacks, so that a caller holding the pair in LDS
// reads each piece only when its matrix instructions need it:
//   qop(cg, kk)        the Q^T operand of column group cg, k-step kk;
//   kop(kk, ka, kb)    the K operands of k-step kk of both blocks;
//   vop(pp, v0, v1)    the V operands of d-tiles 2 pp and 2 pp + 1 (tails masked).
template <int D, int NCG, class QOp, class KOp, class VOp>
__device__ __forceinline__ void attend_pair(const QOp& qop, const KOp& kop, const VOp& vop, bool masked, const int* lim_a,
                                            const int* lim_b, int quad, float c, f32x4_t (&o)[NCG][D / 16],
                                            float* m_run, float* l_lane) {
  f32x4_t sa[NCG], sb[NCG];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    sa[cg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    sb[cg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    uint4 ka, kb;
    kop(kk, ka, kb);
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      const bf16x8_t qk = qop(cg, kk);
      sa[cg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ka), qk, sa[cg], 0, 0, 0);
      sb[cg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kb), qk, sb[cg], 0, 0, 0);
    }
  }
  float mb[NCG];
  bool grow_any = false;
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    if (masked) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (quad * 4 + i >= lim_a[cg]) sa[cg][i] = -INFINITY;
        if (quad * 4 + i >= lim_b[cg]) sb[cg][i] = -INFINITY;
      }
    }
    float m = maxn3(maxn3(sa[cg][0], sa[cg][1], sa[cg][2]), maxn3(sa[cg][3], sb[cg][0], sb[cg][1]),
                    maxn(sb[cg][2], sb[cg][3]));
    m = maxn_xor32(maxn_xor16(m));
    mb[cg] = m * c;
    grow_any |= mb[cg] > m_run[cg] + kRescaleSlack;
  }
  if (__builtin_amdgcn_ballot_w64(grow_any)) {  // wave-uniform branch, rare after the first blocks
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      const float m_new = mb[cg] > m_run[cg] + kRescaleSlack ? mb[cg] : m_run[cg];
      const float alpha = __builtin_amdgcn_exp2f(m_run[cg] - m_new);  // 0 when m_run = -inf, 1 when kept
      l_lane[cg] *= alpha;
#pragma unroll
      for (int i = 0; i < D / 16; ++i) o[cg][i] *= alpha;
      m_run[cg] = m_new;
    }
  }
  bf16x8_t pop[NCG];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    // a masked slot has s = -inf and weight 2^-inf = 0.  A column that has
    // seen no visible key yet keeps m = -inf; it is offset by 0 instead (its
    // slots are all masked then, as any visible one would have raised m)
    const float nm = m_run[cg] == -INFINITY ? 0.f : -m_run[cg];
    float pa[4], pb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pa[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[cg][i], c, nm));
      pb[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sb[cg][i], c, nm));
    }
    l_lane[cg] += ((pa[0] + pa[1]) + (pa[2] + pa[3])) + ((pb[0] + pb[1]) + (pb[2] + pb[3]));
    const bf16x2_t p0 = __builtin_convertvector((f32x2_t{pa[0], pa[1]}), bf16x2_t);
    const bf16x2_t p1 = __builtin_convertvector((f32x2_t{pa[2], pa[3]}), bf16x2_t);
    const bf16x2_t p2 = __builtin_convertvector((f32x2_t{pb[0], pb[1]}), bf16x2_t);
    const bf16x2_t p3 = __builtin_convertvector((f32x2_t{pb[2], pb[3]}), bf16x2_t);
    pop[cg] = __builtin_bit_cast(bf16x8_t, make_uint4(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                                                      __builtin_bit_cast(uint32_t, p2),
                                                      __builtin_bit_cast(uint32_t, p3)));
  }
#pragma unroll
  for (int pp = 0; pp < D / 32; ++pp) {
    uint4 v0, v1;
    vop(pp, v0, v1);
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      o[cg][2 * pp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, v0), pop[cg],
                                                              o[cg][2 * pp], 0, 0, 0);
      o[cg][2 * pp + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, v1), pop[cg],
                                                                  o[cg][2 * pp + 1], 0, 0, 0);
    }
  }
}

// The lane's K and V piece bases of 16-token tile j for a pool of block size
// BS < 16 (16-byte units from the pool base of the layer): the tile gathers
// 16/BS consecutive table entries, and a lane's K pieces lie in the entry of
// its key (lane % 16), its V pieces in the entry of its 4 value slots.  Only
// entries that hold tokens of the context (< n) are read -- the last tile of a
// context may reach past the table's row.  Returns whether a needed entry lies
// outside [0, num_blocks) (such an entry is never dereferenced).  TP: the
// table row's pointer type (a constant-address-space pointer keeps the reads
// scalar where the caller's copies into LDS would otherwise hide that the
// table is read-only).
template <int D, int BS, class TP>
__device__ __forceinline__ bool gather_tile(TP trow, int j, int n, int num_blocks, int n_kv_heads, int g,
                                            int lane, const uint4*& kp, const uint4*& vp, const uint4* kpool,
                                            const uint4* vpool) {
  static_assert(BS == 4 || BS == 8, "a tile gathers entries");
  constexpr int kPer = 16 / BS;
  constexpr int kEntryVec = BS * D * 2 / 16;
  const int quad = lane >> 4, r = lane & 15;
  int pk = 0, pv = 0;
  bool bad = false;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const bool needed = j * 16 + e * BS < n;
    const int ph = needed ? trow[j * kPer + e] : 0;
    const bool b = ph < 0 || ph >= num_blocks;
    bad |= b;
    const int q = b ? 0 : ph;
    pk = r / BS == e ? q : pk;
    pv = quad * 4 / BS == e ? q : pv;
  }
  kp = kpool + (static_cast<int64_t>(pk) * n_kv_heads + g) * kEntryVec + quad * BS + r % BS;
  vp = vpool + (static_cast<int64_t>(pv) * n_kv_heads + g) * kEntryVec + (quad * 4 % BS / 4) * 16 + r;
  return bad;
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
  r.n = min(a.ctx_lens[s], a.max_blocks * a.block_size);
  r.h = r.n - r.c;
  r.bad = r.c > a.max_q_len || (a.causal && r.c > r.n);
  return r;
}

// Keys [0, kend) of tile `tile` of a sequence: up to the position of its last
// column (all n keys without the causal mask).
__device__ __forceinline__ int pf_tile_keys(const pf_args& a, const pf_seq& q, int G, int tile, int nc) {
  if (!a.causal) return q.n;
  const int f_last = min((tile + 1) * nc, q.c * G) - 1;
  return q.h + f_last / G + 1;
}

// BS is the pool's block size B (4 .. 64): for B >= 16, 16-token tile j is
// sub-tile j % (B/16) of table entry j / (B/16), and in the pool's tile layout
// a lane's K pieces of it start at quad * B + lane % 16 + 16 * sub (16-byte
// units inside the entry), its V pieces at lane + 64 * sub, piece i 4 B
// further; for B < 16 a tile gathers 16/B entries (gather_tile).
template <int D, int NCG, int STAGES, int BS = 16>
__global__ void __launch_bounds__(kPfWaves * 64) attn_prefill_kernel(pf_args a) {
  static_assert(BS == 4 || BS == 8 || BS == 16 || BS == 32 || BS == 64, "block size");
  constexpr int kSub = BS >= 16 ? BS / 16 : 1;
  constexpr int NC = 16 * NCG;
  const int lane = threadIdx.x & 63;
  const int quad = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int bid = blockIdx.x;
  const int pg = bid % a.part_groups;
  bid /= a.part_groups;
  const int tg = bid % a.tile_groups;
  bid /= a.tile_groups;
  const int g = bid % a.n_kv_heads;
  const int s = bid / a.n_kv_heads;
  const int G = a.n_q_heads / a.n_kv_heads;
  const int tile = tg * a.wt + wave % a.wt;
  const int part = pg * (kPfWaves / a.wt) + wave / a.wt;

  const pf_seq sq = pf_locate(a, s);
  if (sq.c <= 0 || sq.q0 < 0 || sq.q0 + sq.c > a.total_q) return;  // nothing, or rows outside the output
  const int cols = sq.c * G;
  uint16_t* out = static_cast<uint16_t*>(a.out);
  if (part >= a.max_parts) return;
  if (sq.bad) {  // one wave per unit marks the unit's rows
    if (part == 0 && tile == 0)
      for (int i = lane; i < cols * D; i += 64) {
        const int f = i / D, e = i % D;
        out[(static_cast<int64_t>(sq.q0 + f / G) * a.n_q_heads + g * G + f % G) * D + e] = 0x7fc0;
      }
    return;
  }
  if (tile * NC >= cols) return;
  const int kend = pf_tile_keys(a, sq, G, tile, NC);
  const int P = a.part_blocks * 16;
  const int k_begin = part * P;
  if (k_begin >= kend) return;
  const int n_parts = (kend + P - 1) / P;
  const int b_begin = k_begin >> 4;
  const int b_end = (min(kend, k_begin + P) + 15) >> 4;
  const int f0 = tile * NC;

  // this lane's column in every group; the Q^T operands of the wave's tile
  // go to its LDS slice in operand order (lane l's 16 bytes at l * 16)
  extern __shared__ __align__(16) bf16x8_t pf_q_lds[];
  bf16x8_t* q_lds = pf_q_lds + wave * (NCG * (D / 32) * 64);
  int pos[NCG];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const int f = f0 + cg * 16 + (lane & 15);
    const bool live = f < cols;
    const int j = live ? f / G : 0;
    const int hg = live ? f % G : 0;
    pos[cg] = live ? (a.causal ? sq.h + j : sq.n - 1) : -1;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         (static_cast<int64_t>(sq.q0 + j) * a.n_q_heads + g * G + hg) * D + quad * 8;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
      q_lds[(cg * (D / 32) + kk) * 64 + lane] = live ? *reinterpret_cast<const bf16x8_t*>(qp + kk * 32) : bf16x8_t{};
  }
  // position of the tile's first column: older keys are visible to all
  const int pos_min = a.causal ? sq.h + f0 / G : sq.n - 1;

  const uint4* kpool = static_cast<const uint4*>(a.k_layer);
  const uint4* vpool = static_cast<const uint4*>(a.v_layer);
  constexpr int kEntryVec = BS * D * 2 / 16;  // 16-byte vectors per (entry, kv head)
  const int k_lane = BS == 16 ? lane : quad * BS + (lane & 15);
  const int32_t* trow = a.tables + static_cast<int64_t>(a.table_rows ? a.table_rows[s] : s) * a.max_blocks;
  // ring of STAGES block pairs; loads past the run repeat its last block (L2 hits)
  kv_pair<D> buf[STAGES];
  int phys_a[STAGES], phys_b[STAGES];
  auto issue = [&](int u, int b) {
    const int ja = min(b, b_end - 1), jb = min(b + 1, b_end - 1);
    if constexpr (BS < 16) {
      const uint4 *ka, *va, *kb, *vb;
      phys_a[u] = gather_tile<D, BS>(trow, ja, sq.n, a.num_blocks, a.n_kv_heads, g, lane, ka, va, kpool, vpool) ? -1 : 0;
      phys_b[u] = gather_tile<D, BS>(trow, jb, sq.n, a.num_blocks, a.n_kv_heads, g, lane, kb, vb, kpool, vpool) ? -1 : 0;
      load_pair<D, 4 * BS>(buf[u], ka, va, kb, vb);
      return;
    }
    const int pa = trow[ja / kSub];
    const int pb = trow[jb / kSub];
    phys_a[u] = pa;
    phys_b[u] = pb;
    const int qa = (pa < 0 || pa >= a.num_blocks) ? 0 : pa;  // never dereferenced out of range
    const int qb = (pb < 0 || pb >= a.num_blocks) ? 0 : pb;
    const int64_t ta = (static_cast<int64_t>(qa) * a.n_kv_heads + g) * kEntryVec;
    const int64_t tb = (static_cast<int64_t>(qb) * a.n_kv_heads + g) * kEntryVec;
    const int sa = ja % kSub, sb = jb % kSub;
    load_pair<D, 4 * BS>(buf[u], kpool + ta + 16 * sa + k_lane, vpool + ta + 64 * sa + lane,
                         kpool + tb + 16 * sb + k_lane, vpool + tb + 64 * sb + lane);
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
  const float c = a.scale_log2;

#pragma unroll
  for (int u = 0; u < STAGES; ++u) issue(u, b_begin + 2 * u);
  for (int b0 = b_begin; b0 < b_end; b0 += 2 * STAGES) {
#pragma unroll
    for (int u = 0; u < STAGES; ++u) {
      const int b = b0 + 2 * u;
      // an index that, for all the compiler knows, depends on b keeps the LDS
      // reads of Q^T inside the loop (hoisted, they would hold D/4 * NCG more
      // registers); unlike a memory clobber or a volatile statement it leaves
      // the block-table reads scalar
      int ql;
      asm("" : "=v"(ql) : "0"(lane), "s"(b));
      if (b < b_end) {
        const bool has_b = b + 1 < b_end;  // else the second block is outside the partition: all masked
        const bool bad_a = phys_a[u] < 0 || phys_a[u] >= a.num_blocks;
        const bool bad_b = phys_b[u] < 0 || phys_b[u] >= a.num_blocks;
        poisoned |= bad_a || (has_b && bad_b);
        const int valid_a = bad_a ? 0 : min(16, sq.n - b * 16);
        const int valid_b = (!has_b || bad_b) ? 0 : min(16, sq.n - (b + 1) * 16);
        const v_tail_mask vm(valid_a, valid_b, quad);
        auto qop = [&](int cg, int kk) { return q_lds[(cg * (D / 32) + kk) * 64 + ql]; };
        auto kop = [&](int kk, uint4& ka, uint4& kb) {
          ka = buf[u].ka[kk];
          kb = buf[u].kb[kk];
        };
        auto vop = [&](int pp, uint4& v0, uint4& v1) {
          v0 = vm.apply(buf[u].v[2 * pp]);
          v1 = vm.apply(buf[u].v[2 * pp + 1]);
        };
        // (two specialised steps here: this kernel streams from HBM, and with
        // one step the compiler placed the ring's waits earlier)
        if (valid_a == 16 && valid_b == 16 && b * 16 + 31 <= pos_min) {
          attend_pair<D, NCG>(qop, kop, vop, false, nullptr, nullptr, quad, c, o, m_run, l_lane);
        } else {
          int lim_a[NCG], lim_b[NCG];
#pragma unroll
          for (int cg = 0; cg < NCG; ++cg) {
            lim_a[cg] = min(max(pos[cg] - b * 16 + 1, 0), valid_a);
            lim_b[cg] = min(max(pos[cg] - (b + 1) * 16 + 1, 0), valid_b);
          }
          attend_pair<D, NCG>(qop, kop, vop, true, lim_a, lim_b, quad, c, o, m_run, l_lane);
        }
      }
      issue(u, b + 2 * STAGES);
    }
  }

  const float nan = __builtin_nanf("");
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const float l = sum_xor32(sum_xor16(l_lane[cg]));
    const int f = f0 + cg * 16 + (lane & 15);
    if (f >= cols) continue;
    const int64_t row = static_cast<int64_t>(sq.q0 + f / G) * a.n_q_heads + g * G + f % G;
    if (n_parts == 1 && !a.force_partial) {
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

// ---------------------------------------------------------------------------
// Multi-query attention over a quantised pool (q8_0 / q4_0, B = 16, d <= 128)
// ([INF] §8.4.2: the stored value of a group stands for its code times the
// group's half scale).  The register-ring kernel above with raw tiles in the
// ring: per block pair the codes become exact bf16 operands (codes_block, as
// in the decode kernel), and the scales are applied in float32:
//   score(r, col) = sum_g sK(r, g) * (codes_K(r, group g) . q_col(group g)),
//   O^T          += sum_r  p(r) sV(r, g) codes_V(r, dims of group g),
// so the only rounding beyond float32 is that of each weight p * sV to bf16.
// l sums the unrounded weights.  q4_0 codes carry the bias kQ4Bias: kb[cg][kk]
// (-kQ4Bias times the column's query sum over group kk) starts each score
// product, and every V product is followed by one with the constant operand
// -kQ4Bias on the same weights.
// ---------------------------------------------------------------------------
template <int D, int FMT>
struct kv_qpair {
  kv_qregs<D, FMT> a, b;
};

// One block pair against the NCG column groups: the steps of attend_pair on
// the dequantised pair.  A masked slot (outside the context, or past a
// column's position) gets score -inf and then weight 0 by selection: its
// scale and codes may be anything.
template <int D, int NCG, int FMT, class QOp>
__device__ __forceinline__ void attend_qpair(const QOp& qop, const kv_qpair<D, FMT>& raw,
                                             const float (&kb)[NCG][D / 32], bool masked, const int* lim_a,
                                             const int* lim_b, int quad, float c, f32x4_t (&o)[NCG][D / 16],
                                             float* m_run, float* l_lane) {
  kv_regs<D> ta, tb;
  codes_block<D, FMT>(raw.a, ta);
  codes_block<D, FMT>(raw.b, tb);
  f32x4_t sa[NCG], sb[NCG];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    sa[cg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    sb[cg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      const bf16x8_t qk = qop(cg, kk);
      const f32x4_t b0 = {kb[cg][kk], kb[cg][kk], kb[cg][kk], kb[cg][kk]};
      const f32x4_t xa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ta.k[kk]), qk, b0, 0, 0, 0);
      const f32x4_t xb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, tb.k[kk]), qk, b0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sa[cg][i] = __builtin_fmaf(scale_at<D>(raw.a.ks, i, kk), xa[i], sa[cg][i]);
        sb[cg][i] = __builtin_fmaf(scale_at<D>(raw.b.ks, i, kk), xb[i], sb[cg][i]);
      }
    }
  }
  float mb[NCG];
  bool grow_any = false;
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    if (masked) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (quad * 4 + i >= lim_a[cg]) sa[cg][i] = -INFINITY;
        if (quad * 4 + i >= lim_b[cg]) sb[cg][i] = -INFINITY;
      }
    }
    float m = maxn3(maxn3(sa[cg][0], sa[cg][1], sa[cg][2]), maxn3(sa[cg][3], sb[cg][0], sb[cg][1]),
                    maxn(sb[cg][2], sb[cg][3]));
    m = maxn_xor32(maxn_xor16(m));
    mb[cg] = m * c;
    grow_any |= mb[cg] > m_run[cg] + kRescaleSlack;
  }
  if (__builtin_amdgcn_ballot_w64(grow_any)) {  // wave-uniform branch, rare after the first blocks
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      const float m_new = mb[cg] > m_run[cg] + kRescaleSlack ? mb[cg] : m_run[cg];
      const float alpha = __builtin_amdgcn_exp2f(m_run[cg] - m_new);  // 0 when m_run = -inf, 1 when kept
      l_lane[cg] *= alpha;
#pragma unroll
      for (int i = 0; i < D / 16; ++i) o[cg][i] *= alpha;
      m_run[cg] = m_new;
    }
  }
  float pa[NCG][4], pb[NCG][4];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const float nm = m_run[cg] == -INFINITY ? 0.f : -m_run[cg];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pa[cg][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[cg][i], c, nm));
      pb[cg][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sb[cg][i], c, nm));
    }
    l_lane[cg] += ((pa[cg][0] + pa[cg][1]) + (pa[cg][2] + pa[cg][3])) +
                  ((pb[cg][0] + pb[cg][1]) + (pb[cg][2] + pb[cg][3]));
  }
  // O^T += V^T . (P * sV)^T over the 32 tokens of the pair, one weight operand
  // per group of 32 dims (d-tiles 2 pp and 2 pp + 1); the V operand of d-tile
  // t is block a's 4 slots of the lane then block b's (as kv_pair::v)
#pragma unroll
  for (int pp = 0; pp < D / 32; ++pp) {
    const uint4 v0 = make_uint4(ta.v[pp].x, ta.v[pp].y, tb.v[pp].x, tb.v[pp].y);
    const uint4 v1 = make_uint4(ta.v[pp].z, ta.v[pp].w, tb.v[pp].z, tb.v[pp].w);
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      float w[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w[i] = __builtin_fmaf(scale_at<D>(raw.a.vs, i, pp), pa[cg][i], 0.f);
        w[4 + i] = __builtin_fmaf(scale_at<D>(raw.b.vs, i, pp), pb[cg][i], 0.f);
      }
      if (masked) {  // wave uniform
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          w[i] = pa[cg][i] == 0.f ? 0.f : w[i];
          w[4 + i] = pb[cg][i] == 0.f ? 0.f : w[4 + i];
        }
      }
      const bf16x8_t pop = __builtin_bit_cast(
          bf16x8_t, make_uint4(pack_bf16x2(w[0], w[1]), pack_bf16x2(w[2], w[3]), pack_bf16x2(w[4], w[5]),
                               pack_bf16x2(w[6], w[7])));
      o[cg][2 * pp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, v0), pop, o[cg][2 * pp],
                                                              0, 0, 0);
      o[cg][2 * pp + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, v1), pop,
                                                                  o[cg][2 * pp + 1], 0, 0, 0);
      if constexpr (FMT == kFmtQ4) {
        const bf16x8_t nb = __builtin_bit_cast(bf16x8_t, make_uint4(kQ4NegBiasPair, kQ4NegBiasPair, kQ4NegBiasPair,
                                                                    kQ4NegBiasPair));
        o[cg][2 * pp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(nb, pop, o[cg][2 * pp], 0, 0, 0);
        o[cg][2 * pp + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(nb, pop, o[cg][2 * pp + 1], 0, 0, 0);
      }
    }
  }
}

// The register-ring multi-query kernel over a quantised pool: work split,
// queries in LDS, masks, partials and output exactly as attn_prefill_kernel;
// the ring holds STAGES raw block pairs (codes and scales of K and V).  Two
// waves per SIMD: the code conversion and scaling are vector work that one
// wave's own dependency chains leave idle; the launch takes one column group
// per wave (the registers of two column groups do not fit beside a second wave).
template <int D, int NCG, int FMT, int STAGES>
__global__ void __launch_bounds__(kPfWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) attn_prefill_q_kernel(pf_args a) {
  static_assert(FMT == kFmtQ8 || FMT == kFmtQ4, "quantised pools");
  static_assert(D <= 128, "d <= 128");
  constexpr int NC = 16 * NCG;
  const int lane = threadIdx.x & 63;
  const int quad = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int bid = blockIdx.x;
  const int pg = bid % a.part_groups;
  bid /= a.part_groups;
  const int tg = bid % a.tile_groups;
  bid /= a.tile_groups;
  const int g = bid % a.n_kv_heads;
  const int s = bid / a.n_kv_heads;
  const int G = a.n_q_heads / a.n_kv_heads;
  const int tile = tg * a.wt + wave % a.wt;
  const int part = pg * (kPfWaves / a.wt) + wave / a.wt;

  const pf_seq sq = pf_locate(a, s);
  if (sq.c <= 0 || sq.q0 < 0 || sq.q0 + sq.c > a.total_q) return;  // nothing, or rows outside the output
  const int cols = sq.c * G;
  uint16_t* out = static_cast<uint16_t*>(a.out);
  if (part >= a.max_parts) return;
  if (sq.bad) {  // one wave per unit marks the unit's rows
    if (part == 0 && tile == 0)
      for (int i = lane; i < cols * D; i += 64) {
        const int f = i / D, e = i % D;
        out[(static_cast<int64_t>(sq.q0 + f / G) * a.n_q_heads + g * G + f % G) * D + e] = 0x7fc0;
      }
    return;
  }
  if (tile * NC >= cols) return;
  const int kend = pf_tile_keys(a, sq, G, tile, NC);
  const int P = a.part_blocks * 16;
  const int k_begin = part * P;
  if (k_begin >= kend) return;
  const int n_parts = (kend + P - 1) / P;
  const int b_begin = k_begin >> 4;
  const int b_end = (min(kend, k_begin + P) + 15) >> 4;
  const int f0 = tile * NC;

  // the Q^T operands of the wave's tile to its LDS slice in operand order,
  // and for q4_0 each column's bias term per group of 32 dims (the lane holds
  // 8 of the group's dims; the four quads hold the rest)
  extern __shared__ __align__(16) bf16x8_t pf_q_lds[];
  bf16x8_t* q_lds = pf_q_lds + wave * (NCG * (D / 32) * 64);
  int pos[NCG];
  float kb[NCG][D / 32];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const int f = f0 + cg * 16 + (lane & 15);
    const bool live = f < cols;
    const int j = live ? f / G : 0;
    const int hg = live ? f % G : 0;
    pos[cg] = live ? (a.causal ? sq.h + j : sq.n - 1) : -1;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         (static_cast<int64_t>(sq.q0 + j) * a.n_q_heads + g * G + hg) * D + quad * 8;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      const bf16x8_t qv = live ? *reinterpret_cast<const bf16x8_t*>(qp + kk * 32) : bf16x8_t{};
      q_lds[(cg * (D / 32) + kk) * 64 + lane] = qv;
      kb[cg][kk] = 0.f;
      if constexpr (FMT == kFmtQ4) {
        const uint4 w = __builtin_bit_cast(uint4, qv);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
        float part_sum = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          part_sum += __uint_as_float(ws[k] << 16) + __uint_as_float(ws[k] & 0xffff0000u);
        kb[cg][kk] = -kQ4Bias * sum_xor32(sum_xor16(part_sum));
      }
    }
  }
  const int pos_min = a.causal ? sq.h + f0 / G : sq.n - 1;

  const unsigned char* kbase = static_cast<const unsigned char*>(a.k_layer);
  const unsigned char* vbase = static_cast<const unsigned char*>(a.v_layer);
  constexpr int64_t kTileBytes = q_tile_bytes<D, FMT>();
  const int32_t* trow = a.tables + static_cast<int64_t>(a.table_rows ? a.table_rows[s] : s) * a.max_blocks;
  // ring of STAGES raw block pairs; loads past the run repeat its last block (L2 hits)
  kv_qpair<D, FMT> buf[STAGES];
  int phys_a[STAGES], phys_b[STAGES];
  auto issue = [&](int u, int b) {
    const int pa = trow[min(b, b_end - 1)];
    const int pb = trow[min(b + 1, b_end - 1)];
    phys_a[u] = pa;
    phys_b[u] = pb;
    const int qa = (pa < 0 || pa >= a.num_blocks) ? 0 : pa;  // never dereferenced out of range
    const int qb = (pb < 0 || pb >= a.num_blocks) ? 0 : pb;
    const int64_t ta = (static_cast<int64_t>(qa) * a.n_kv_heads + g) * kTileBytes;
    const int64_t tb = (static_cast<int64_t>(qb) * a.n_kv_heads + g) * kTileBytes;
    load_qblock<D, FMT>(buf[u].a, kbase + ta, vbase + ta, lane);
    load_qblock<D, FMT>(buf[u].b, kbase + tb, vbase + tb, lane);
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
  const float c = a.scale_log2;

#pragma unroll
  for (int u = 0; u < STAGES; ++u) issue(u, b_begin + 2 * u);
  for (int b0 = b_begin; b0 < b_end; b0 += 2 * STAGES) {
#pragma unroll
    for (int u = 0; u < STAGES; ++u) {
      const int b = b0 + 2 * u;
      // (an index the compiler takes to depend on b keeps the LDS reads of
      // Q^T inside the loop, as in attn_prefill_kernel)
      int ql;
      asm("" : "=v"(ql) : "0"(lane), "s"(b));
      if (b < b_end) {
        const bool has_b = b + 1 < b_end;  // else the second block is outside the partition: all masked
        const bool bad_a = phys_a[u] < 0 || phys_a[u] >= a.num_blocks;
        const bool bad_b = phys_b[u] < 0 || phys_b[u] >= a.num_blocks;
        poisoned |= bad_a || (has_b && bad_b);
        const int valid_a = bad_a ? 0 : min(16, sq.n - b * 16);
        const int valid_b = (!has_b || bad_b) ? 0 : min(16, sq.n - (b + 1) * 16);
        auto qop = [&](int cg, int kk) { return q_lds[(cg * (D / 32) + kk) * 64 + ql]; };
        if (valid_a == 16 && valid_b == 16 && b * 16 + 31 <= pos_min) {
          attend_qpair<D, NCG, FMT>(qop, buf[u], kb, false, nullptr, nullptr, quad, c, o, m_run, l_lane);
        } else {
          int lim_a[NCG], lim_b[NCG];
#pragma unroll
          for (int cg = 0; cg < NCG; ++cg) {
            lim_a[cg] = min(max(pos[cg] - b * 16 + 1, 0), valid_a);
            lim_b[cg] = min(max(pos[cg] - (b + 1) * 16 + 1, 0), valid_b);
          }
          attend_qpair<D, NCG, FMT>(qop, buf[u], kb, true, lim_a, lim_b, quad, c, o, m_run, l_lane);
        }
      }
      issue(u, b + 2 * STAGES);
    }
  }

  const float nan = __builtin_nanf("");
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const float l = sum_xor32(sum_xor16(l_lane[cg]));
    const int f = f0 + cg * 16 + (lane & 15);
    if (f >= cols) continue;
    const int64_t row = static_cast<int64_t>(sq.q0 + f / G) * a.n_q_heads + g * G + f % G;
    if (n_parts == 1 && !a.force_partial) {
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

// The same attention with the K/V of each block pair shared through LDS by the
// WT waves of a partition group (consecutive tiles of one unit, one partition):
// the group's waves copy disjoint 1 KiB chunks of the pair (K and V tiles of
// both blocks) from global memory straight into an S-slot LDS ring
// (global_load_lds, no registers), and every wave reads the whole pair from
// there.  Each pair crosses the L2 -> CU path once per group instead of once
// per wave, S - 1 pairs are in flight per group, and the registers hold only
// Q^T, the accumulators and the pair being consumed.
// Pipeline per pair k: wait until this wave's chunks of pair k have landed
// (s_waitcnt on the vector-memory counter, which counts the copies in order);
// barrier (everyone's chunks of pair k are in, and everyone has finished
// reading slot (k-1) mod S); issue the copies of pair k + S - 1 into that
// slot; read pair k and attend.  Every iteration issues the same number of
// copies (past the group's last pair they repeat it into a slot nobody reads)
// so the wait count is a constant.  The loop count is uniform over the
// workgroup (the largest partition of its groups); a wave with no columns or
// no keys left copies and waits but does not attend.  D <= 128.
// BS: the pool's block size (4 .. 64), as for attn_prefill_kernel; the
// copies put every 16-token tile into its slot in the B = 16 order.
template <int D, int NCG, int WT, int S, int BS = 16>
__global__ void __launch_bounds__(kPfWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_prefill_lds_kernel(pf_args a) {
  static_assert(BS == 4 || BS == 8 || BS == 16 || BS == 32 || BS == 64, "block size");
  constexpr int kSub = BS >= 16 ? BS / 16 : 1;
  constexpr int kEntryVec = BS * D * 2 / 16;  // 16-byte vectors per (entry, kv head)
  constexpr int NC = 16 * NCG;
  constexpr int kTileVec = 16 * D * 2 / 16;    // 16-byte vectors per K or V tile
  constexpr int kChunks = 4 * kTileVec / 64;   // 1 KiB chunks per pair: Ka, Kb, Va, Vb
  constexpr int kMine = kChunks / WT;          // chunks this wave copies
  constexpr int kGroups = kPfWaves / WT;       // partition groups per workgroup
  static_assert(kChunks % WT == 0, "chunks split evenly");
  static_assert(S >= 2 && (S - 2) * kMine <= 63, "the wait count fits the vector-memory counter");
  const int lane = threadIdx.x & 63;
  const int quad = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int bid = blockIdx.x;
  const int pgi = bid % a.part_groups;
  bid /= a.part_groups;
  const int tg = bid % a.tile_groups;
  bid /= a.tile_groups;
  const int g = bid % a.n_kv_heads;
  const int s = bid / a.n_kv_heads;
  const int G = a.n_q_heads / a.n_kv_heads;
  const int tw = wave % WT;    // tile within the workgroup
  const int grp = wave / WT;   // partition group within the workgroup
  const int tile = tg * WT + tw;
  const int part = pgi * kGroups + grp;

  // exits taken by the whole workgroup (they depend on s and tg only)
  const pf_seq sq = pf_locate(a, s);
  if (sq.c <= 0 || sq.q0 < 0 || sq.q0 + sq.c > a.total_q) return;
  const int cols = sq.c * G;
  uint16_t* out = static_cast<uint16_t*>(a.out);
  if (sq.bad) {
    if (pgi == 0 && tg == 0 && wave == 0)
      for (int i = lane; i < cols * D; i += 64) {
        const int f = i / D, e = i % D;
        out[(static_cast<int64_t>(sq.q0 + f / G) * a.n_q_heads + g * G + f % G) * D + e] = 0x7fc0;
      }
    return;
  }
  const int n_tiles = (cols + NC - 1) / NC;
  if (tg * WT >= n_tiles) return;
  const int P = a.part_blocks * 16;
  // the workgroup's last tile sees the most keys: its groups load up to there
  const int kend_wg = pf_tile_keys(a, sq, G, min(tg * WT + WT, n_tiles) - 1, NC);
  auto group_pairs = [&](int pt) __attribute__((always_inline)) {  // pairs group partition pt loads
    if (pt >= a.max_parts || pt * P >= kend_wg) return 0;
    const int nb = ((min(kend_wg, pt * P + P) + 15) >> 4) - ((pt * P) >> 4);
    return (nb + 1) >> 1;
  };
  int n_iter = 0;
#pragma unroll
  for (int gg = 0; gg < kGroups; ++gg) n_iter = max(n_iter, group_pairs(pgi * kGroups + gg));
  if (n_iter == 0) return;
  const int my_pairs = group_pairs(part);
  const int b_begin = (part * P) >> 4;
  const int grp_b_end = my_pairs > 0 ? ((min(kend_wg, part * P + P) + 15) >> 4) : b_begin;

  // this wave's own tile: keys, block range, partition count
  const bool live_tile = tile < n_tiles && part < a.max_parts;
  const int kend = live_tile ? pf_tile_keys(a, sq, G, tile, NC) : 0;
  const bool computes = live_tile && part * P < kend;
  const int b_end = computes ? ((min(kend, part * P + P) + 15) >> 4) : b_begin;
  const int n_parts = (kend + P - 1) / P;
  const int f0 = tile * NC;

  // Q^T operands of the wave's columns, in registers
  bf16x8_t qreg[NCG][D / 32];
  int pos[NCG];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const int f = f0 + cg * 16 + (lane & 15);
    const bool live = computes && f < cols;
    const int j = live ? f / G : 0;
    const int hg = live ? f % G : 0;
    pos[cg] = live ? (a.causal ? sq.h + j : sq.n - 1) : -1;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         (static_cast<int64_t>(sq.q0 + j) * a.n_q_heads + g * G + hg) * D + quad * 8;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
      qreg[cg][kk] = live ? *reinterpret_cast<const bf16x8_t*>(qp + kk * 32) : bf16x8_t{};
  }
  const int pos_min = a.causal ? sq.h + f0 / G : sq.n - 1;

  const uint4* kpool = static_cast<const uint4*>(a.k_layer);
  const uint4* vpool = static_cast<const uint4*>(a.v_layer);
  // the table row through the constant address space: read-only for the
  // kernel's lifetime, so its (uniform) entries stay scalar loads even though
  // the copies into LDS write memory the compiler cannot tell apart from it
  typedef const __attribute__((address_space(4))) int32_t ctable_t;
  ctable_t* trow = (ctable_t*)(a.tables + static_cast<int64_t>(a.table_rows ? a.table_rows[s] : s) * a.max_blocks);
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  extern __shared__ __align__(16) u32x4_t pf_kv_lds[];
  u32x4_t* ring = pf_kv_lds + grp * S * (kChunks * 64);  // this group's S slots

  // copies of pair kp (clamped to the group's last pair; block 0 of the head
  // for a group with no pair) into slot kp mod S.  Chunk c of a pair: tile
  // c / (D/32) (0 Ka, 1 Kb, 2 Va, 3 Vb), 1 KiB piece c % (D/32).
  auto copy_pair = [&](int kp) __attribute__((always_inline)) {
    if constexpr (BS < 16) {
      // every lane's pieces from the entries its key and value slots lie in
      const uint4 *ka = kpool, *va = vpool, *kb = kpool, *vb = vpool;
      if (my_pairs > 0) {
        const int b = b_begin + 2 * min(kp, my_pairs - 1);
        const int ja = min(b, grp_b_end - 1), jb = min(b + 1, grp_b_end - 1);
        gather_tile<D, BS>(trow, ja, sq.n, a.num_blocks, a.n_kv_heads, g, lane, ka, va, kpool, vpool);
        gather_tile<D, BS>(trow, jb, sq.n, a.num_blocks, a.n_kv_heads, g, lane, kb, vb, kpool, vpool);
      }
      u32x4_t* slot = ring + (kp % S) * (kChunks * 64);
#pragma unroll
      for (int j = 0; j < kMine; ++j) {
        const int c = tw + j * WT;
        const int t = c / (D / 32), i = c % (D / 32);
        const uint4* base = t == 0 ? ka : (t == 1 ? kb : (t == 2 ? va : vb));
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(base + i * 4 * BS),
                                         (__attribute__((address_space(3))) void*)(slot + c * 64), 16, 0, 0);
      }
      return;
    }
    int qa = 0, qb = 0, sa = 0, sb = 0;
    if (my_pairs > 0) {
      const int b = b_begin + 2 * min(kp, my_pairs - 1);
      const int ja = min(b, grp_b_end - 1), jb = min(b + 1, grp_b_end - 1);
      const int pa = trow[ja / kSub];
      const int pb = trow[jb / kSub];
      qa = (pa < 0 || pa >= a.num_blocks) ? 0 : pa;  // never dereferenced out of range
      qb = (pb < 0 || pb >= a.num_blocks) ? 0 : pb;
      sa = ja % kSub;
      sb = jb % kSub;
    }
    const int64_t ta = (static_cast<int64_t>(qa) * a.n_kv_heads + g) * kEntryVec;
    const int64_t tb = (static_cast<int64_t>(qb) * a.n_kv_heads + g) * kEntryVec;
    u32x4_t* slot = ring + (kp % S) * (kChunks * 64);
#pragma unroll
    for (int j = 0; j < kMine; ++j) {
      const int c = tw + j * WT;
      const int t = c / (D / 32), i = c % (D / 32);
      // the lane's 16-byte piece i of tile t (Ka, Kb, Va, Vb): for B = 16 one
      // 1 KiB run per piece; for B > 16 the sub-tile's piece in the entry
      const uint4* src;
      if constexpr (BS == 16) {
        src = (t < 2 ? kpool : vpool) + ((t & 1) ? tb : ta) + i * 64 + lane;
      } else {
        const int sub = (t & 1) ? sb : sa;
        src = t < 2 ? kpool + ((t & 1) ? tb : ta) + 16 * sub + i * 4 * BS + quad * BS + (lane & 15)
                    : vpool + ((t & 1) ? tb : ta) + 64 * sub + i * 4 * BS + lane;
      }
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src),
                                       (__attribute__((address_space(3))) void*)(slot + c * 64), 16, 0, 0);
    }
  };
  // s_waitcnt vmcnt(n), the other counters untouched
  constexpr int kWait = (S - 2) * kMine;
  constexpr int kVmWait = (kWait & 15) | ((kWait >> 4) << 14) | (7 << 4) | (15 << 8);
  constexpr int kVmDrain = (7 << 4) | (15 << 8);

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
  const float c = a.scale_log2;
  auto qop = [&](int cg, int kk) __attribute__((always_inline)) { return qreg[cg][kk]; };
  // The V operands of a pair take the two blocks' halves side by side, so
  // each lane reads them as four 8-byte pieces straight into place.  The high
  // halves go through an offset of 8 that the compiler cannot see through;
  // otherwise it merges each two 8-byte reads back into one 16-byte read and
  // then moves the halves into the operands with one instruction per dword.
  int hi8;
  asm("v_mov_b32 %0, 8" : "=v"(hi8));

#pragma unroll
  for (int kp = 0; kp < S - 1; ++kp) copy_pair(kp);
  for (int k = 0; k < n_iter; ++k) {
    __builtin_amdgcn_s_waitcnt(kVmWait);  // this wave's chunks of pair k have landed
    __builtin_amdgcn_s_barrier();         // everyone's have; slot (k - 1) mod S is free
    copy_pair(k + S - 1);
    const int b = b_begin + 2 * k;
    const bool mine = b < b_end;
    if (mine) {
      const u32x4_t* sl = ring + (k % S) * (kChunks * 64);
      const bool has_b = b + 1 < b_end;
      bool bad_a, bad_b;
      if constexpr (BS < 16) {
        const uint4 *k0, *v0;
        bad_a = gather_tile<D, BS>(trow, b, sq.n, a.num_blocks, a.n_kv_heads, g, lane, k0, v0, kpool, vpool);
        bad_b = gather_tile<D, BS>(trow, min(b + 1, b_end - 1), sq.n, a.num_blocks, a.n_kv_heads, g, lane, k0, v0,
                                   kpool, vpool);
      } else {
        const int pa = trow[b / kSub];
        const int pb = trow[min(b + 1, b_end - 1) / kSub];
        bad_a = pa < 0 || pa >= a.num_blocks;
        bad_b = pb < 0 || pb >= a.num_blocks;
      }
      poisoned |= bad_a || (has_b && bad_b);
      const int valid_a = bad_a ? 0 : min(16, sq.n - b * 16);
      const int valid_b = (!has_b || bad_b) ? 0 : min(16, sq.n - (b + 1) * 16);
      // only a pair reaching past the context has V slots to clear
      const bool vtail = valid_a < 16 || valid_b < 16;
      // operands read from the slot when the matrix instructions need them
      auto kop = [&](int kk, uint4& ka, uint4& kb) __attribute__((always_inline)) {
        const u32x4_t x = sl[(0 * (D / 32) + kk) * 64 + lane];
        const u32x4_t y = sl[(1 * (D / 32) + kk) * 64 + lane];
        ka = make_uint4(x[0], x[1], x[2], x[3]);
        kb = make_uint4(y[0], y[1], y[2], y[3]);
      };
      // (the slot is read through the same pointer type the copies write, or
      // the compiler makes the reads wait for every copy in flight.  The tail
      // branch is wave uniform; the empty asm keeps it a branch rather than
      // per-dword selects on every pair)
      auto vop = [&](int pp, uint4& v0, uint4& v1) __attribute__((always_inline)) {
        const char* va = reinterpret_cast<const char*>(sl + (2 * (D / 32) + pp) * 64 + lane);
        const char* vb = reinterpret_cast<const char*>(sl + (3 * (D / 32) + pp) * 64 + lane);
        const u32x2_t a0 = *reinterpret_cast<const u32x2_t*>(va), b0 = *reinterpret_cast<const u32x2_t*>(vb);
        const u32x2_t a1 = *reinterpret_cast<const u32x2_t*>(va + hi8);
        const u32x2_t b1 = *reinterpret_cast<const u32x2_t*>(vb + hi8);
        v0 = make_uint4(a0[0], a0[1], b0[0], b0[1]);
        v1 = make_uint4(a1[0], a1[1], b1[0], b1[1]);
        if (vtail) {
          int va_n = valid_a, vb_n = valid_b;  // defined here, so the mask's compares stay in the branch
          asm volatile("" : "+s"(va_n), "+s"(vb_n));
          const v_tail_mask vm(va_n, vb_n, quad);
          v0 = vm.apply(v0);
          v1 = vm.apply(v1);
          asm volatile("" : "+v"(v0.x), "+v"(v0.y), "+v"(v0.z), "+v"(v0.w));
          asm volatile("" : "+v"(v1.x), "+v"(v1.y), "+v"(v1.z), "+v"(v1.w));
        }
      };
      const bool masked = valid_a < 16 || valid_b < 16 || b * 16 + 31 > pos_min;
      int lim_a[NCG], lim_b[NCG];
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) {
        lim_a[cg] = min(max(pos[cg] - b * 16 + 1, 0), valid_a);
        lim_b[cg] = min(max(pos[cg] - (b + 1) * 16 + 1, 0), valid_b);
      }
      attend_pair<D, NCG>(qop, kop, vop, masked, lim_a, lim_b, quad, c, o, m_run, l_lane);
    }
  }
  // the last copies (repeats nobody reads) must land before the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(kVmDrain);
  if (!computes) return;

  const float nan = __builtin_nanf("");
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const float l = sum_xor32(sum_xor16(l_lane[cg]));
    const int f = f0 + cg * 16 + (lane & 15);
    if (f >= cols) continue;
    const int64_t row = static_cast<int64_t>(sq.q0 + f / G) * a.n_q_heads + g * G + f % G;
    if (n_parts == 1 && !a.force_partial) {
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
// one carries NaN into the row.  One wave per (row, head): lane p holds the
// weight of partition p (64 at a time), then every lane accumulates its
// dimensions over the partitions.
constexpr int kPfMergeWaves = 4;
constexpr int kPfMergeBatch = 8;  // partial rows per batch of loads

template <int D>
__global__ void __launch_bounds__(kPfMergeWaves * 64) merge_prefill_kernel(pf_args a) {
  const int lane = threadIdx.x & 63;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * kPfMergeWaves + (threadIdx.x >> 6);
  if (item >= static_cast<int64_t>(a.total_q) * a.n_q_heads) return;
  const int r = static_cast<int>(item / a.n_q_heads);
  const int head = static_cast<int>(item % a.n_q_heads);
  // sequence of row r: the last s with q_indptr[s] <= r; the lanes test 64
  // sequences at a time and count the passes (q_indptr is non-decreasing)
  int passed = 0;
  for (int base = 0; base < a.n_seqs; base += 64) {
    const int s = base + lane;
    const uint64_t ok = __builtin_amdgcn_ballot_w64(s < a.n_seqs && a.q_indptr[s] <= r);
    passed += __builtin_popcountll(ok);
    if (ok != ~0ull) break;
  }
  const pf_seq sq = pf_locate(a, max(passed - 1, 0));
  if (sq.c <= 0 || r < sq.q0 || r >= sq.q0 + sq.c || sq.bad) return;
  const int G = a.n_q_heads / a.n_kv_heads;
  const int f = (r - sq.q0) * G + head % G;
  const int kend = pf_tile_keys(a, sq, G, f / a.cols_per_tile, a.cols_per_tile);
  const int P = a.part_blocks * 16;
  const int n_parts = (kend + P - 1) / P;
  if (n_parts <= 1) return;
  const int64_t base = item * a.max_parts;
  constexpr int E = (D + 63) / 64;  // dims per lane
  uint16_t* orow = static_cast<uint16_t*>(a.out) + item * D;
  if (n_parts <= 64) {
    // the usual case: lane p holds partition p's (m, l), read once, and the
    // rows are loaded kPfMergeBatch at a time with no branch between the
    // loads (rows of weight 0 are loaded but not added)
    const float m = lane < n_parts ? a.part_m[base + lane] : -INFINITY;
    const float l = lane < n_parts ? a.part_l[base + lane] : 0.f;
    const bool nan_seen = __builtin_amdgcn_ballot_w64(m != m) != 0;
    const float M = wave_max(m != m ? -INFINITY : m);
    const float w = (m == -INFINITY || m != m) ? 0.f : exp2f(m - M);
    const float L = wave_sum(w == 0.f ? 0.f : w * l);
    float acc[E];
#pragma unroll
    for (int i = 0; i < E; ++i) acc[i] = 0.f;
    for (int k0 = 0; k0 < n_parts; k0 += kPfMergeBatch) {
      float v[kPfMergeBatch][E];
#pragma unroll
      for (int k = 0; k < kPfMergeBatch; ++k) {
        const float* po = a.part_o + (base + min(k0 + k, n_parts - 1)) * D;
#pragma unroll
        for (int i = 0; i < E; ++i) v[k][i] = lane + 64 * i < D ? po[lane + 64 * i] : 0.f;
      }
#pragma unroll
      for (int k = 0; k < kPfMergeBatch; ++k) {
        const float wk = k0 + k < n_parts ? __shfl(w, k0 + k) : 0.f;
#pragma unroll
        for (int i = 0; i < E; ++i) acc[i] = wk == 0.f ? acc[i] : __builtin_fmaf(wk, v[k][i], acc[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < E; ++i)
      if (lane + 64 * i < D) orow[lane + 64 * i] = f32_to_bf16(nan_seen ? __builtin_nanf("") : acc[i] / L);
    return;
  }
  float M = -INFINITY;
  bool nan_seen = false;
  for (int p0 = 0; p0 < n_parts; p0 += 64) {
    const float m = p0 + lane < n_parts ? a.part_m[base + p0 + lane] : -INFINITY;
    nan_seen |= __builtin_amdgcn_ballot_w64(m != m) != 0;
    M = fmaxf(M, m);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  float acc[E];
#pragma unroll
  for (int i = 0; i < E; ++i) acc[i] = 0.f;
  float L = 0.f;
  for (int p0 = 0; p0 < n_parts; p0 += 64) {
    const int p = p0 + lane;
    const float m = p < n_parts ? a.part_m[base + p] : -INFINITY;
    const float w = (m == -INFINITY || m != m) ? 0.f : exp2f(m - M);
    L += w == 0.f ? 0.f : w * a.part_l[base + p];
    const int np = min(64, n_parts - p0);
    for (int k = 0; k < np; ++k) {
      const float wk = __shfl(w, k);
      if (wk == 0.f) continue;  // wave uniform
      const float* po = a.part_o + (base + p0 + k) * D;
#pragma unroll
      for (int i = 0; i < E; ++i)
        if (lane + 64 * i < D) acc[i] += wk * po[lane + 64 * i];
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o);
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
  int wt;           // tiles per workgroup
  int tile_groups;  // workgroups per unit along tiles
  int part_groups;  // workgroups per unit along partitions
  int partition;    // tokens per partition
  int max_parts;
  float scale;
};

// LDS of one CU on the current device.
int64_t max_lds_per_cu() {
  static int bytes = -1;
  if (bytes < 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&bytes, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess ||
        bytes <= 0)
      bytes = 65536;
  }
  return bytes;
}

// The pools the multi-query kernels read: bf16 with B in {4, 8, 16, 32, 64} and d in
// {64, 128, 256}; q8_0 / q4_0 with B = 16 and d in {64, 128}; G <= 16.
bool pf_supported(const kv_pool_config& c, int G) {
  if (G < 1 || G > kMaxGroup || (c.head_dim != 64 && c.head_dim != 128 && c.head_dim != 256)) return false;
  if (c.dtype == KV_BF16)
    return c.block_size == 4 || c.block_size == 8 || c.block_size == 16 || c.block_size == 32 || c.block_size == 64;
  return is_quantized(c.dtype) && c.block_size == 16 && c.head_dim <= 128;
}

kv_status pf_resolve(const kv_pool* pool, int n_seqs, int total_q, int max_q_len, int num_q_heads, int max_blocks,
                     const kv_attention_options* opts, pf_plan& p) {
  if (!pool) return fail(KV_ERR_INVALID, "pool is NULL");
  const kv_pool_config& c = pool->cfg;
  if (num_q_heads <= 0 || num_q_heads % c.num_kv_heads != 0)
    return fail(KV_ERR_INVALID, "num_q_heads must be a positive multiple of num_kv_heads");
  const int G = num_q_heads / c.num_kv_heads;
  if (n_seqs < 0 || total_q < 0 || max_blocks <= 0 || max_q_len <= 0)
    return fail(KV_ERR_INVALID, "n_seqs, total_q >= 0 and max_q_len, max_blocks_per_seq > 0 required");
  kv_attention_options o{0.f, 0, KV_KERNEL_AUTO, nullptr};
  if (opts) o = *opts;
  if (o.kernel != KV_KERNEL_AUTO && o.kernel != KV_KERNEL_MFMA)
    return fail(KV_ERR_UNSUPPORTED, "multi-query attention has only the matrix-core kernel");
  const bool quant = is_quantized(c.dtype);
  if (!pf_supported(c, G))
    return fail(KV_ERR_UNSUPPORTED, "the multi-query kernels need G <= 16 and bf16 with B in {4, 8, 16, 32, 64}, d in {64, "
                                    "128, 256}, or q8_0 / q4_0 with B = 16, d in {64, 128}");
  if (o.partition_tokens < 0 || o.partition_tokens % 16 != 0)
    return fail(KV_ERR_INVALID, "partition_tokens must be 0 or a positive multiple of the block size");
  if (!(o.scale >= 0.f) || std::isinf(o.scale)) return fail(KV_ERR_INVALID, "scale must be finite and >= 0");
  p.scale = o.scale > 0.f ? o.scale : 1.f / std::sqrt(static_cast<float>(c.head_dim));
  const int64_t cols = static_cast<int64_t>(max_q_len) * G;
  // 16-column groups per wave: two when there are enough columns for several
  // two-group tiles (the LDS-sharing kernel then reads each pair from LDS once
  // per 32 columns instead of 16); one otherwise, and at d = 256
  p.ncg = (c.head_dim <= 128 && cols > 64 && !quant) ? 2 : 1;
  p.tiles = static_cast<int>((cols + 16 * p.ncg - 1) / (16 * p.ncg));
  p.wt = p.tiles >= 4 ? 4 : (p.tiles >= 2 ? 2 : 1);
  p.tile_groups = (p.tiles + p.wt - 1) / p.wt;
  const int64_t max_ctx = static_cast<int64_t>(max_blocks) * c.block_size;
  if (o.partition_tokens > 0) {
    p.partition = o.partition_tokens;
  } else {
    // enough waves to fill the CUs once: the LDS-sharing kernel (several
    // tiles per partition, d <= 128) runs as many workgroups per CU as its
    // ring allows, at most two; the register-ring kernel two waves per SIMD.
    // Beyond that, one partition per tile.
    const int64_t waves = static_cast<int64_t>(n_seqs) * c.num_kv_heads * p.tiles;
    int64_t want = 8LL * device_cus();
    if (p.wt >= 2 && c.head_dim <= 128 && !quant) {
      const int64_t ring = static_cast<int64_t>(kPfWaves / p.wt) * (p.wt == 2 ? 3 : 4) * 4 * 16 * c.head_dim * 2;
      const int64_t per_cu = std::max<int64_t>(1, std::min<int64_t>(2, max_lds_per_cu() / ring));
      want = kPfWaves * per_cu * device_cus();
    }
    if (waves >= want) {
      p.partition = static_cast<int>(max_ctx);
    } else {
      const int64_t parts = (want + std::max<int64_t>(waves, 1) - 1) / std::max<int64_t>(waves, 1);
      const int64_t per = ((max_ctx + parts - 1) / parts + 15) / 16 * 16;
      p.partition = static_cast<int>(std::max<int64_t>(256, per));
    }
  }
  p.max_parts = static_cast<int>((max_ctx + p.partition - 1) / p.partition);
  const int wp = kPfWaves / p.wt;
  p.part_groups = (p.max_parts + wp - 1) / wp;
  const int64_t grid = static_cast<int64_t>(n_seqs) * c.num_kv_heads * p.tile_groups * p.part_groups;
  if (grid > 0x7fffffff) return fail(KV_ERR_INVALID, "grid too large");
  return KV_OK;
}

uint64_t pf_workspace(const kv_pool_config& c, int total_q, int num_q_heads, const pf_plan& p) {
  if (p.max_parts <= 1) return 0;
  const uint64_t rows = static_cast<uint64_t>(total_q) * num_q_heads * p.max_parts;
  return 2 * up256(rows * 4) + up256(rows * c.head_dim * 4);
}

// Ring depth in block pairs: the wider tiles hold more accumulators and fewer
// blocks in flight.
template <int D, int NCG, int BS>
hipError_t pf_launch(const pf_args& a, int64_t grid, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  constexpr size_t kPair = 4 * 16 * D * 2;  // Ka, Kb, Va, Vb
  // several tiles per partition: share each block pair through LDS; ring
  // depth 4 pairs for one partition group (64 KiB at d = 128, two workgroups
  // per CU), 3 for two groups (96 KiB, one workgroup per CU)
  if constexpr (D <= 128) {
    if (a.wt == 2 && (kPfWaves / 2) * 3 * kPair <= max_lds_per_block()) {
      return launch_timed(attn_prefill_lds_kernel<D, NCG, 2, 3, BS>, dim3(static_cast<unsigned>(grid)),
                          dim3(kPfWaves * 64), (kPfWaves / 2) * 3 * kPair, st, ev0, ev1, a);
    }
    if (a.wt == 4 && (kPfWaves / 4) * 4 * kPair <= max_lds_per_block()) {
      return launch_timed(attn_prefill_lds_kernel<D, NCG, 4, 4, BS>, dim3(static_cast<unsigned>(grid)),
                          dim3(kPfWaves * 64), (kPfWaves / 4) * 4 * kPair, st, ev0, ev1, a);
    }
  }
  constexpr int kStages = D >= 256 ? 1 : 2;
  constexpr size_t kLds = static_cast<size_t>(kPfWaves) * NCG * (D / 32) * 64 * 16;  // Q^T operands per wave
  return launch_timed(attn_prefill_kernel<D, NCG, kStages, BS>, dim3(static_cast<unsigned>(grid)), dim3(kPfWaves * 64),
                      static_cast<uint32_t>(kLds), st, ev0, ev1, a);
}

// Quantised pools: the register-ring kernel with raw tiles, one column group
// per wave, two waves per SIMD; ring depth 2 pairs (1 at d = 128).
template <int D, int NCG, int FMT>
hipError_t pf_launch_q(const pf_args& a, int64_t grid, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  constexpr size_t kLds = static_cast<size_t>(kPfWaves) * NCG * (D / 32) * 64 * 16;  // Q^T operands per wave
  return launch_timed(attn_prefill_q_kernel<D, NCG, FMT, D >= 128 ? 1 : 2>, dim3(static_cast<unsigned>(grid)), dim3(kPfWaves * 64),
                      static_cast<uint32_t>(kLds), st, ev0, ev1, a);
}

template <int D>
hipError_t pf_launch_d(const pf_args& a, int ncg, int32_t dtype, int64_t grid, hipStream_t st, hipEvent_t ev0,
                       hipEvent_t ev1) {
  if constexpr (D <= 128) {
    if (dtype == KV_Q8_0) return pf_launch_q<D, 1, kFmtQ8>(a, grid, st, ev0, ev1);
    if (dtype == KV_Q4_0) return pf_launch_q<D, 1, kFmtQ4>(a, grid, st, ev0, ev1);
  }
  if (dtype != KV_BF16) return hipErrorInvalidValue;
  if (ncg == 1) {
    switch (a.block_size) {
      case 4: return pf_launch<D, 1, 4>(a, grid, st, ev0, ev1);
      case 8: return pf_launch<D, 1, 8>(a, grid, st, ev0, ev1);
      case 16: return pf_launch<D, 1, 16>(a, grid, st, ev0, ev1);
      case 32: return pf_launch<D, 1, 32>(a, grid, st, ev0, ev1);
      case 64: return pf_launch<D, 1, 64>(a, grid, st, ev0, ev1);
      default: return hipErrorInvalidValue;
    }
  }
  if constexpr (D <= 128) {
    if (ncg == 2) {
      switch (a.block_size) {
        case 4: return pf_launch<D, 2, 4>(a, grid, st, ev0, ev1);
        case 8: return pf_launch<D, 2, 8>(a, grid, st, ev0, ev1);
        case 16: return pf_launch<D, 2, 16>(a, grid, st, ev0, ev1);
        case 32: return pf_launch<D, 2, 32>(a, grid, st, ev0, ev1);
        case 64: return pf_launch<D, 2, 64>(a, grid, st, ev0, ev1);
        default: return hipErrorInvalidValue;
      }
    }
  }
  return hipErrorInvalidValue;
}

template <int D>
hipError_t pf_merge(const pf_args& a, hipStream_t st, hipEvent_t ev1) {
  const int64_t items = static_cast<int64_t>(a.total_q) * a.n_q_heads;
  const int64_t grid = (items + kPfMergeWaves - 1) / kPfMergeWaves;
  return launch_timed(merge_prefill_kernel<D>, dim3(static_cast<unsigned>(grid)), dim3(kPfMergeWaves * 64), 0u, st,
                      nullptr, ev1, a);
}

// Whether a call goes to the row-wise path (one decode query per chunk row):
// the generic kernel asked for, or a pool the multi-query kernels do not read
// (f32, other block sizes, quantised at d = 256).
bool rowwise(const kv_pool* pool, int num_q_heads, const kv_attention_options* opts) {
  if (!pool || num_q_heads <= 0 || num_q_heads % pool->cfg.num_kv_heads != 0) return false;
  const int G = num_q_heads / pool->cfg.num_kv_heads;
  if (opts && opts->kernel == KV_KERNEL_GENERIC) return true;
  return !pf_supported(pool->cfg, G);
}

}  // namespace

}  // namespace pagedkv

using namespace pagedkv;

extern "C" {

uint64_t paged_prefill_workspace_bytes(const kv_pool* pool, int32_t n_seqs, int32_t total_q, int32_t max_q_len,
                                       int32_t num_q_heads, int32_t max_blocks_per_seq,
                                       const kv_attention_options* opts) {
  if (rowwise(pool, num_q_heads, opts)) {
    if (n_seqs < 0 || total_q < 0 || max_q_len <= 0 || max_blocks_per_seq <= 0) return 0;
    return prefill_rowwise_workspace(pool, total_q, num_q_heads, max_blocks_per_seq, opts);
  }
  pf_plan p;
  if (pf_resolve(pool, n_seqs, total_q, max_q_len, num_q_heads, max_blocks_per_seq, opts, p) != KV_OK) return 0;
  return pf_workspace(pool->cfg, total_q, num_q_heads, p);
}

kv_status paged_attention_prefill(kv_pool* pool, int32_t layer, const void* q, void* out, const int32_t* d_q_indptr,
                                  const int32_t* d_block_tables, const int32_t* d_context_lens, int32_t n_seqs,
                                  int32_t total_q, int32_t max_q_len, int32_t max_blocks_per_seq,
                                  int32_t num_q_heads, const kv_attention_options* opts, void* d_workspace,
                                  uint64_t workspace_bytes, void* hip_stream) {
  if (rowwise(pool, num_q_heads, opts)) {
    const kv_pool_config& c = pool->cfg;
    if (layer < 0 || layer >= c.num_layers) return fail(KV_ERR_INVALID, "layer out of range");
    if (n_seqs < 0 || total_q < 0 || max_q_len <= 0 || max_blocks_per_seq <= 0)
      return fail(KV_ERR_INVALID, "n_seqs, total_q >= 0 and max_q_len, max_blocks_per_seq > 0 required");
    if (n_seqs == 0 || total_q == 0) return KV_OK;
    if (!q || !out || !d_q_indptr || !d_block_tables || !d_context_lens || !pool->k_cache || !pool->v_cache)
      return fail(KV_ERR_INVALID, "NULL device pointer");
    if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out)) & 15)
      return fail(KV_ERR_INVALID, "q and out must be 16-byte aligned");
    return prefill_rowwise(pool, layer, q, out, d_q_indptr, d_block_tables, d_context_lens, n_seqs, total_q,
                           max_q_len, max_blocks_per_seq, num_q_heads, opts, d_workspace, workspace_bytes,
                           static_cast<hipStream_t>(hip_stream));
  }
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
      static_cast<int64_t>(layer) * c.num_blocks * c.num_kv_heads * tile_bytes(c);
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
  a.wt = p.wt;
  a.tile_groups = p.tile_groups;
  a.part_groups = p.part_groups;
  a.cols_per_tile = 16 * p.ncg;
  a.block_size = c.block_size;
  a.scale_log2 = p.scale * kLog2e;
  a.causal = 1;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const int64_t grid = static_cast<int64_t>(n_seqs) * c.num_kv_heads * p.tile_groups * p.part_groups;
  const call_events ev = events_of(opts);
  hipError_t e;
  switch (c.head_dim) {
    case 64: e = pf_launch_d<64>(a, p.ncg, c.dtype, grid, st, ev.start, ev.kernel_stop); break;
    case 128: e = pf_launch_d<128>(a, p.ncg, c.dtype, grid, st, ev.start, ev.kernel_stop); break;
    default: e = pf_launch_d<256>(a, p.ncg, c.dtype, grid, st, ev.start, ev.kernel_stop); break;
  }
  if (kv_status s = hip_check(e, "paged_attention_prefill launch")) return s;
  if (p.max_parts > 1) {
    switch (c.head_dim) {
      case 64: e = pf_merge<64>(a, st, ev.stop); break;
      case 128: e = pf_merge<128>(a, st, ev.stop); break;
      default: e = pf_merge<256>(a, st, ev.stop); break;
    }
    return hip_check(e, "paged_attention_prefill merge launch");
  }
  if (ev.stop) return hip_check(hipEventRecord(ev.stop, st), "timing event");
  return KV_OK;
}

}  // extern "C"
