// Read-once decode over shared prefixes ("cascade") for gfx950: one persistent
// matrix-core launch that streams every group's shared prefix once and every
// member's own blocks once, then one merge.
//
// Sequences come in groups [group_start[g], group_start[g+1]) whose tables
// agree on their first shared[g] blocks (forks of one request; [KVM]
// copy-on-write branching and cross-turn prefix caching make such blocks
// physically shared).  The decode of a member splits its keys in two ranges,
// folded with the running-max recurrences of [KVM] (chunked prefill
// mechanism).  The work is one list of units:
//   prefix units: (group, chunk of members, kv head).  The shared tiles are
//     read once and multiplied by the queries of all members of the chunk at
//     once -- up to 4 column tiles of 16 (members x G query heads), whose
//     operands stay in registers for the whole unit;
//   suffix units: (member, kv head), the member's blocks past the shared
//     ones, one column tile (its G query heads).
// The list is cut into contiguous runs, one per wave of the persistent grid,
// by cost rather than by tile count (a prefix tile costs more than a suffix
// tile, and every unit a run starts costs a little), and every wave streams
// its run through one register ring.  Every run writes partials (m, l, O)
// where it ends inside a unit; cascade_merge_kernel folds, per (member, query
// head), the partials of its prefix unit and of its suffix unit.
//
// Over a quantised pool (q8_0 / q4_0) the ring holds raw tiles and the codes
// feed the matrix instructions, the group scales applied in float32 ([INF]
// §8.4.2); a prefix unit then carries 2 column tiles instead of 4.
//
// The contract is checked on the device: a member whose shared table entries
// differ from the first member's (compared tile by tile as the prefix
// streams), whose context or whose first member's context does not cover
// the prefix, or whose group is larger than max_group or malformed, gets a NaN
// row; so does a member reading a table entry outside [0, N).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <limits>
#include <string>
#include <type_traits>

#include "device_common.h"
#include "pool_internal.h"

namespace pagedkv {
namespace {

constexpr int kCsWaves = 4;  // waves per workgroup, one per SIMD

// Column tiles of a prefix unit: 4 (64 query columns) up to d = 128, 2 at
// d = 256 (register budget of one wave per SIMD); over a quantised pool half
// as many (the raw tiles and their conversion take the registers).
template <int D, int FMT>
constexpr int cs_tiles() {
  return (D <= 128 ? 4 : 2) / (FMT == kFmtBf16 ? 1 : 2);
}
inline int cs_tiles_rt(int d, int32_t dtype) { return (d <= 128 ? 4 : 2) / (dtype == KV_BF16 ? 1 : 2); }

// Register-ring depth: the deepest whose registers fit beside the accumulators
// of the column tiles and a suffix unit's queries (qpl 16-byte pieces per
// lane), with no spills.
__host__ __device__ constexpr int cs_stages(int d, int qpl) {
  return d >= 256 ? 2 : (d == 128 ? (qpl >= 4 ? 2 : 3) : 6);
}

struct cs_args {
  const void* q;
  void* out;
  const void* k_layer;
  const void* v_layer;
  const int32_t* tables;
  const int32_t* ctx_lens;
  const int32_t* group_start;
  const int32_t* shared;
  float* a_m;  // prefix partials: row = slot * acol + column, slot = wave + unit
  float* a_l;
  float* a_o;  // [..][D]
  float* b_m;  // suffix partials: row = (slot - n_a Hkv) * G + head in group
  float* b_l;
  float* b_o;
  int32_t* cum_parts;  // [n_a + n_seqs + 1] partitions before each item, per kv head (workgroup 0 writes)
  int32_t* cum_cost;   // [n_a + n_seqs + 1] work-split cost before each item, per kv head (workgroup 0 writes)
  int4* member;    // [n_seqs]: prefix tiles (-1: NaN row), prefix item (-1: none), first column, 0
  int4* mdesc;     // [n_seqs][Hkv]: first wave and wave count of the member's prefix unit, then of its
                   // suffix unit (workgroup 0 writes, for the merge)
  int n_seqs, n_groups, cpg, mc, max_group, max_blocks, n_q_heads, n_kv_heads, num_blocks, part_blocks, n_waves;
  int acol;                // columns of a prefix unit's partial rows (column tiles x 16)
  int wa, wb, wu;          // work-split cost of a prefix partition, a suffix partition, a unit's start
  int aslot, bslot;        // elements of a wave's prefix and suffix query slots
  int aslot2;              // elements of a wave's second prefix slot (0: none)
  float scale_log2;
};

// LDS ints of the plan over V items (n_a prefix chunks, then n members) of
// ng groups: cum_t, cum_p, cum_c (V + 1 each), ctx_n and j0 (n each), the
// group starts (ng + 1), rounded up to 16 bytes; the staged queries follow.
__host__ __device__ constexpr int cs_lds_ints(int V, int n, int ng) { return (3 * (V + 1) + 2 * n + ng + 1 + 3) & ~3; }

// Sum of x over lanes 0 .. l of the wave, at lane l (every lane active): DPP
// row shifts by 1, 2, 4 and 8 within each 16-lane row (lanes shifted in from
// outside the row read 0), then each row adds the totals of the rows before
// it, read from lanes 15, 31 and 47.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31);
  const int r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}

// In place over cum_b (tiles per item on entry): exclusive prefix sums of the
// tiles, of the partitions ceil(tiles / pb) and of the work-split cost
// (partitions x wa for the first na items, x wb after, plus wu for an item
// with partitions) into cum_b, cum_p and cum_c, totals at index n.  Every
// thread of the workgroup takes part.
__device__ void cs_scan(int* cum_b, int* cum_p, int* cum_c, int n, int pb, int na, int wa, int wb, int wu) {
  __shared__ int wsum[3][kCsWaves];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int carry_b = 0, carry_p = 0, carry_c = 0;
  for (int base = 0; base < n; base += kCsWaves * 64) {
    const int i = base + tid;
    const int t = i < n ? cum_b[i] : 0;
    const int p = (t + pb - 1) / pb;
    const int c = p > 0 ? p * (i < na ? wa : wb) + wu : 0;
    const int ib = wave_incl_scan(t), ip = wave_incl_scan(p), ic = wave_incl_scan(c);
    if (lane == 63) {
      wsum[0][wv] = ib;
      wsum[1][wv] = ip;
      wsum[2][wv] = ic;
    }
    __syncthreads();
    int before_b = carry_b, before_p = carry_p, before_c = carry_c;
    for (int k = 0; k < wv; ++k) {
      before_b += wsum[0][k];
      before_p += wsum[1][k];
      before_c += wsum[2][k];
    }
    if (i < n) {
      cum_b[i] = before_b + ib - t;
      cum_p[i] = before_p + ip - p;
      cum_c[i] = before_c + ic - c;
    }
    for (int k = 0; k < kCsWaves; ++k) {
      carry_b += wsum[0][k];
      carry_p += wsum[1][k];
      carry_c += wsum[2][k];
    }
    __syncthreads();
  }
  if (tid == 0) {
    cum_b[n] = carry_b;
    cum_p[n] = carry_p;
    cum_c[n] = carry_c;
  }
  __syncthreads();
}

// The split of the work list among the waves.  The partitions are numbered
// item by item (prefix chunks first), kv head by kv head within an item; a
// unit (item, kv head) costs wu to start and wa per prefix partition or wb
// per suffix partition (a prefix tile is attended by up to 64 query columns,
// a suffix tile by G; starting a unit stages queries and ends another one's
// run), so partition k of a unit starts k ? wu + k w : 0 into the unit.
// Wave w takes the partitions whose starting cost lies in
// [floor(w C / W), floor((w + 1) C / W)), C the total.  When a wave's share
// would be below the largest gap between two starts (wu + max(wa, wb)), the
// cost is the partition count instead (and waves past the partitions get
// none); otherwise every wave gets work.
struct cs_split {
  bool weighted;
  int64_t C, W;
  int wa, wb, wu, na, Hkv;
  __device__ cs_split(const int32_t* cum_p, const int32_t* cum_c, int V, int na_, int Hkv_, int wa_, int wb_, int wu_,
                      int64_t W_)
      : W(W_), wa(wa_), wb(wb_), wu(wu_), na(na_), Hkv(Hkv_) {
    const int64_t cc = static_cast<int64_t>(Hkv) * cum_c[V];
    weighted = cc >= W * (wu + max(wa, wb));
    C = weighted ? cc : static_cast<int64_t>(Hkv) * cum_p[V];
  }
  // starting cost of partition k of unit (item, kvh); cb = cost before the
  // item per kv head, uc = the item's cost per kv head
  __device__ int64_t start(int item, int kvh, int k, int64_t cb, int64_t uc) const {
    const int w = item < na ? wa : wb;
    return static_cast<int64_t>(Hkv) * cb + kvh * uc + (weighted ? (k ? wu + static_cast<int64_t>(k) * w : 0) : k);
  }
  // the wave that takes a partition starting at cost st
  __device__ int64_t owner(int64_t st) const { return div_nn((st + 1) * W - 1, C); }
  // with item (whose cost range holds c), its partitions np, costs before cb
  // and per kv head uc, partitions before pb: the first partition (global
  // index) whose starting cost is >= c
  __device__ int64_t first_at(int64_t c, int item, int np, int64_t cb, int64_t uc, int64_t pb) const {
    const int64_t r = c - static_cast<int64_t>(Hkv) * cb;
    const int64_t h = div_nn(r, uc), r2 = r - h * uc;
    int64_t k;
    if (weighted) {
      const int w = item < na ? wa : wb;
      k = r2 == 0 ? 0 : (r2 <= wu ? 1 : div_nn(r2 - wu + w - 1, w));
    } else {
      k = r2;
    }
    return static_cast<int64_t>(Hkv) * pb + h * np + min<int64_t>(k, np);
  }
};

// Uniform reads of the tables and the group starts go through the constant
// address space: both are read-only for the kernel's lifetime, so the reads
// stay scalar loads even though the kernel writes memory the compiler cannot
// tell apart from them.  (A vector load there would be waited for with every
// tile load issued before it -- a drain of the whole register ring.)
typedef const __attribute__((address_space(4))) int32_t cint_t;

__device__ __forceinline__ int cload(const int32_t* p, int64_t i) { return ((cint_t*)p)[i]; }

// Entry jt of table row trow (-1 for a row < 0).
__device__ __forceinline__ int tables_entry(const int32_t* tables, int trow, int max_blocks, int64_t jt) {
  return trow >= 0 ? cload(tables, static_cast<int64_t>(trow) * max_blocks + jt) : -1;
}

// Position of a wave's run: space (0 = prefix units, 1 = suffix units), item,
// kv head, tile j of the unit (relative to its first tile j0), the unit's
// tiles nb, its table row, first tile, context tokens and, for a prefix unit,
// the first member of its chunk and the chunk's member count.  Wave uniform.
struct cs_cursor {
  int sp, item, kvh, j, nb, trow, j0, n, m0, cnt;
};

// FMT: bf16, or a quantised pool (q8_0 / q4_0) read as in the decode kernel --
// the ring holds raw tiles, whose codes become exact bf16 operands per tile;
// each 32-dim group's score product is scaled by its K scale in float32 and
// each V group's weights by its V scale ([INF] §8.4.2).
template <int D, int STAGES, int QPL, int FMT = kFmtBf16>
__global__ void __launch_bounds__(kCsWaves * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
attn_cascade_kernel(cs_args a) {
  constexpr int NT = cs_tiles<D, FMT>();
  extern __shared__ __align__(16) int cs_smem[];
  const int n = a.n_seqs;
  const int na = a.n_groups * a.cpg;
  const int V = na + n;  // items: the prefix chunks, then the members' suffixes
  int* cum_t = cs_smem;          // [V + 1] tiles before each item, per kv head
  int* cum_p = cum_t + V + 1;    // [V + 1] partitions before each item, per kv head
  int* cum_c = cum_p + V + 1;    // [V + 1] work-split cost before each item, per kv head
  int* ctx_n = cum_c + V + 1;    // [n] clamped context tokens
  int* j0s = ctx_n + n;          // [n] first tile of each member's suffix (-1: NaN row)
  int* gsl = j0s + n;            // [n_groups + 1] group starts
  __shared__ int malformed;
  const int G = a.n_q_heads / a.n_kv_heads;
  const int Hkv = a.n_kv_heads;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int quad = lane >> 4;
  const int col16 = lane & 15;
  const int cap = a.max_blocks * 16;
  const bool publish = blockIdx.x == 0;  // workgroup 0 writes the plan for the merge

  // ---- the plan: which members read which prefix, and every unit's tiles ----
  // The first loop reads every global input of the plan (contexts, group
  // starts, shared block counts) into LDS, all independent loads, so the plan
  // waits out one memory latency; the rest works in LDS.  gst (in cum_c until
  // the scan) holds the group starts; gS (in cum_p until the scan) each
  // group's shared blocks, then its prefix tiles, -1 for a group whose
  // members get NaN rows; j0s holds each member's group until it holds its
  // prefix tiles.
  int* gS = cum_p;
  int* gst = cum_c;
  for (int s = tid; s < max(n, a.n_groups + 1); s += kCsWaves * 64) {
    if (s < n) {
      j0s[s] = -1;
      ctx_n[s] = max(min(a.ctx_lens[s], cap), 0);
    }
    if (s <= a.n_groups) gst[s] = gsl[s] = a.group_start[s];
    if (s < a.n_groups) gS[s] = a.shared[s];
  }
  for (int v = tid; v < na; v += kCsWaves * 64) cum_t[v] = 0;  // prefix tiles per chunk
  if (tid == 0) malformed = 0;
  __syncthreads();
  for (int g = tid; g < a.n_groups; g += kCsWaves * 64) {
    const int first = gst[g], end = gst[g + 1];
    const bool well = first >= 0 && end <= n && first <= end && (g > 0 || first == 0) &&
                      (g < a.n_groups - 1 || end == n);
    if (!well) malformed = 1;  // every member gets a NaN row
    const int S = gS[g];
    const bool ok = well && first < end && end - first <= a.max_group && S >= 0 && S <= a.max_blocks &&
                    16 * S <= ctx_n[first];
    gS[g] = ok ? S : -1;
    if (well)
      for (int s = first; s < end; ++s) j0s[s] = g;  // LDS only
    if (ok)
      for (int c = 0; c < a.cpg; ++c) cum_t[g * a.cpg + c] = (S > 0 && c * a.mc < end - first) ? S : 0;
  }
  __syncthreads();
  const bool bad_plan = malformed != 0;
  if (bad_plan)
    for (int v = tid; v < na; v += kCsWaves * 64) cum_t[v] = 0;
  // each thread reads and rewrites only its own members' entries
  for (int s = tid; s < n; s += kCsWaves * 64) {
    const int g = bad_plan ? -1 : j0s[s];
    const int S = g >= 0 ? gS[g] : -1;
    const bool covers = S >= 0 && 16 * S <= ctx_n[s];
    const int first = g >= 0 ? gst[g] : 0;
    const int4 r = make_int4(covers ? S : -1, covers && S > 0 ? g * a.cpg + (s - first) / a.mc : -1,
                             ((s - first) % a.mc) * G, 0);
    j0s[s] = r.x;
    cum_t[na + s] = r.x >= 0 ? max((ctx_n[s] + 15) / 16 - r.x, 0) : 0;  // suffix tiles
    if (publish) a.member[s] = r;
  }
  __syncthreads();
  cs_scan(cum_t, cum_p, cum_c, V, a.part_blocks, na, a.wa, a.wb, a.wu);
  if (publish)
    for (int v = tid; v <= V; v += kCsWaves * 64) {
      a.cum_parts[v] = cum_p[v];
      a.cum_cost[v] = cum_c[v];
    }

  auto rfl = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
  const int64_t wid = static_cast<int64_t>(blockIdx.x) * kCsWaves + wave;
  const int64_t W = a.n_waves;
  const cs_split split(cum_p, cum_c, V, na, Hkv, a.wa, a.wb, a.wu, W);
  const int* cum_x = split.weighted ? cum_c : cum_p;  // the split's cost before each item
  // the first partition whose starting cost is >= c (the item is the last one
  // whose cost range starts at or before c: the lanes test 64 items at a time)
  auto first_at = [&](int64_t c) __attribute__((always_inline)) -> int64_t {
    if (c >= split.C) return static_cast<int64_t>(Hkv) * rfl(cum_p[V]);
    int passed = 0;
    for (int base = 0; base < V; base += 64) {
      const int i = base + lane;
      const bool ok = i < V && static_cast<int64_t>(Hkv) * cum_x[i] <= c;
      const uint64_t m = __builtin_amdgcn_ballot_w64(ok);
      passed += __builtin_popcountll(m);
      if (m != ~0ull) break;
    }
    const int item = max(passed - 1, 0);
    const int np = rfl(cum_p[item + 1]) - rfl(cum_p[item]);
    const int cb = rfl(cum_x[item]);
    return split.first_at(c, item, np, cb, rfl(cum_x[item + 1]) - cb, rfl(cum_p[item]));
  };
  if (publish) {
    // for the merge: the waves holding each (member, kv head)'s prefix unit
    // and suffix unit (the members as loop 3 wrote them: same workgroup,
    // after the barriers above)
    auto waves_of = [&](int item, int kvh, int& w0, int& cnt) {
      const int np = cum_p[item + 1] - cum_p[item];
      w0 = 0;
      cnt = 0;
      if (np <= 0) return;
      const int64_t cb = cum_x[item], uc = cum_x[item + 1] - cb;
      const int64_t f = split.owner(split.start(item, kvh, 0, cb, uc));
      w0 = static_cast<int>(f);
      cnt = static_cast<int>(split.owner(split.start(item, kvh, np - 1, cb, uc)) - f + 1);
    };
    for (int i = tid; i < n * Hkv; i += kCsWaves * 64) {
      const int s = i / Hkv, kvh = i % Hkv;
      const int4 mi = a.member[s];
      int4 d = make_int4(0, 0, 0, 0);
      if (mi.x > 0 && mi.y >= 0) waves_of(mi.y, kvh, d.x, d.y);
      if (mi.x >= 0) waves_of(na + s, kvh, d.z, d.w);
      a.mdesc[i] = d;
    }
  }
  const int64_t p_begin = first_at(div_nn(wid * split.C, W)), p_end = first_at(div_nn((wid + 1) * split.C, W));
  if (p_begin >= p_end) return;

  // unit data that depends on the item
  auto fill_unit = [&](cs_cursor& c) __attribute__((always_inline)) {
    c.nb = rfl(cum_t[c.item + 1]) - rfl(cum_t[c.item]);
    if (c.item < na) {
      const int g = c.item / a.cpg, ch = c.item % a.cpg;
      const int first = rfl(gsl[g]), end = rfl(gsl[g + 1]);
      c.sp = 0;
      c.trow = first;
      c.j0 = 0;
      c.n = 16 * c.nb;
      c.m0 = first + ch * a.mc;
      c.cnt = min(a.mc, end - c.m0);
    } else {
      const int s = c.item - na;
      c.sp = 1;
      c.trow = s;
      c.j0 = rfl(j0s[s]);
      c.n = rfl(ctx_n[s]);
      c.m0 = s;
      c.cnt = 1;
    }
  };
  // partition index -> cursor (the item is the last one whose first partition
  // is <= pp: the lanes test 64 items at a time)
  auto locate = [&](int64_t pp, cs_cursor& c) __attribute__((always_inline)) {
    int passed = 0;
    for (int base = 0; base < V; base += 64) {
      const int i = base + lane;
      const bool ok = i < V && static_cast<int64_t>(Hkv) * cum_p[i] <= pp;
      const uint64_t m = __builtin_amdgcn_ballot_w64(ok);
      passed += __builtin_popcountll(m);
      if (m != ~0ull) break;
    }
    c.item = max(passed - 1, 0);
    const int np = rfl(cum_p[c.item + 1]) - rfl(cum_p[c.item]);
    const int64_t r = pp - static_cast<int64_t>(Hkv) * rfl(cum_p[c.item]);
    const int64_t h = div_nn(r, np);
    c.kvh = static_cast<int>(h);
    c.j = static_cast<int>(r - h * np) * a.part_blocks;
    fill_unit(c);
  };
  auto flat = [&](const cs_cursor& c) __attribute__((always_inline)) -> int64_t {
    return static_cast<int64_t>(Hkv) * rfl(cum_t[c.item]) + static_cast<int64_t>(c.kvh) * c.nb + c.j;
  };
  cs_cursor first, last;
  locate(p_begin, first);
  locate(p_end - 1, last);
  last.j = min(last.j + a.part_blocks, last.nb) - 1;
  const int n_blk = static_cast<int>(flat(last) - flat(first)) + 1;  // tiles of this run
  // step a cursor to the next tile
  auto advance = [&](cs_cursor& c) __attribute__((always_inline)) {
    if (++c.j < c.nb) return;
    c.j = 0;
    if (++c.kvh < Hkv) return;
    c.kvh = 0;
    do {
      ++c.item;
    } while (c.item < V - 1 && rfl(cum_t[c.item + 1]) == rfl(cum_t[c.item]));
    fill_unit(c);
  };

  const uint4* kpool = static_cast<const uint4*>(a.k_layer);
  const uint4* vpool = static_cast<const uint4*>(a.v_layer);
  constexpr int kTileVec = 16 * D * 2 / 16;

  // ---- staged queries -------------------------------------------------
  // A wave holds two LDS slots: the queries of its current prefix unit (up to
  // mc members x G heads) and those of its current suffix unit (G heads).
  // The first prefix unit of a run is copied before the ring is first filled;
  // a later one (rare: prefix units are long) when it starts, waiting for
  // everything in flight.  A suffix unit's G x D queries travel as ordinary
  // loads into registers (QPL 16-byte pieces per lane, carried by the ring
  // stage of the unit's first tile), issued by the load side just before that
  // tile's loads -- so the wait for them is the tile's own -- and written to
  // the suffix slot when that tile is consumed.
  uint16_t* a_slot = reinterpret_cast<uint16_t*>(cs_smem + cs_lds_ints(V, n, a.n_groups)) +
                     static_cast<int64_t>(wave) * (a.aslot + a.aslot2 + a.bslot);
  uint16_t* a_slot2 = a_slot + a.aslot;  // the next prefix unit's, when a run reaches into it
  uint16_t* b_slot = a_slot2 + a.aslot2;
  // columns sit kQStride = D + 8 elements apart: the 16 lanes of a quarter
  // wave read 16 consecutive columns, which a stride of D would put in one
  // LDS bank (a 16-way conflict on every operand read)
  constexpr int kQStride = D + 8;
  auto padded = [](int e) __attribute__((always_inline)) { return (e / D) * kQStride + e % D; };
  // copies the first prefix unit's query columns (member-major: column
  // m * G + h) to its slot before the ring is first filled: every piece is
  // loaded (at most NT x 16 columns, 16 pieces per lane up to d = 256), then
  // all are written, so the copy waits out one memory latency.  (Copies
  // straight from global memory to LDS are avoided everywhere in this kernel:
  // the compiler would then make every LDS read wait for all loads.)
  auto stage_prefix = [&](const cs_cursor& c, uint16_t* dst) __attribute__((always_inline)) {
    const uint16_t* qg = static_cast<const uint16_t*>(a.q);
    const int elems = c.cnt * G * D;  // <= NT x 16 columns
    constexpr int kPieces = NT * 16 * D / 512;
    // the piece of lane `lane` at element offset (i * 64 + lane) * 8
    auto src = [&](int e) __attribute__((always_inline)) {
      const int col = e / D, dim = e % D;
      const int m = col / G, h = col % G;
      return reinterpret_cast<const uint4*>(qg + (static_cast<int64_t>(c.m0 + m) * a.n_q_heads + c.kvh * G + h) * D +
                                            dim);
    };
    uint4 v[kPieces];
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const int e = (i * 64 + lane) * 8;
      v[i] = e < elems ? *src(e) : uint4{};
    }
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const int e = (i * 64 + lane) * 8;
      if (e < elems) *reinterpret_cast<uint4*>(dst + padded(e)) = v[i];
    }
  };

  // ---- load side: STAGES tiles ahead of consumption (the last one repeats
  // past the end of the run and is served by the L2) ----
  cs_cursor ld = first;
  int ld_k = 0;
  bool ld_new = true;  // the load cursor is at the first tile of a unit of the run
  bool bad_ring[STAGES];  // the tile's table entry lies outside [0, N)
  int phys_ring[STAGES];  // the entry itself (prefix tiles: compared with the members' entries)
  int chk_ring[STAGES];   // prefix tiles: lane i < cnt holds member m0 + i's entry of the tile
  // a ring stage: the tile's K/V operands and, when a suffix unit starts at
  // the tile, the unit's queries
  using ring_t = typename std::conditional<FMT == kFmtBf16, kv_regs<D>, kv_qregs<D, FMT>>::type;
  struct stage_regs {
    ring_t kv;
    uint4 q[QPL];
  };
  // the table entry of the tile at cursor c; the caller reads it and hands it
  // to issue (the first STAGES are read together before the ring is first
  // filled, so the fill waits out one memory latency instead of one per tile)
  auto entry_of = [&](const cs_cursor& c) __attribute__((always_inline)) {
    return tables_entry(a.tables, c.trow, a.max_blocks, static_cast<int64_t>(c.j0) + c.j);
  };
  auto issue = [&](stage_regs& sr, int u, int phys) __attribute__((always_inline)) {
    if (ld_new && ld.sp == 1) {
      const uint4* qg = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) +
                                                       (static_cast<int64_t>(ld.m0) * a.n_q_heads + ld.kvh * G) * D);
#pragma unroll
      for (int i = 0; i < QPL; ++i)
        if ((i * 64 + lane) * 8 < G * D) sr.q[i] = qg[i * 64 + lane];
    }
    ld_new = false;
    const int64_t jt = ld.j0 + ld.j;
    const bool bad = phys < 0 || phys >= a.num_blocks;
    bad_ring[u] = bad;
    phys_ring[u] = phys;
    if (ld.sp == 0 && lane < ld.cnt)
      chk_ring[u] = a.tables[static_cast<int64_t>(ld.m0 + lane) * a.max_blocks + jt];
    const int p = bad ? 0 : phys;  // never dereferenced out of range
    if constexpr (FMT == kFmtBf16) {
      const int64_t t = (static_cast<int64_t>(p) * Hkv + ld.kvh) * kTileVec;
      load_block<D>(sr.kv, kpool + t, vpool + t, lane);
    } else {
      const int64_t t = (static_cast<int64_t>(p) * Hkv + ld.kvh) * q_tile_bytes<D, FMT>();
      load_qblock<D, FMT>(sr.kv, static_cast<const unsigned char*>(a.k_layer) + t,
                          static_cast<const unsigned char*>(a.v_layer) + t, lane);
    }
    if (++ld_k < n_blk) {
      const int item = ld.item, kvh = ld.kvh;
      advance(ld);
      ld_new = ld.item != item || ld.kvh != kvh;
    }
  };

  // the table entries of the first ring fill, read together (and before the
  // queries are staged, so that the two memory latencies overlap)
  int pre[STAGES];
  {
    cs_cursor c = ld;
#pragma unroll
    for (int u = 0; u < STAGES; ++u) {
      pre[u] = entry_of(c);
      if (u + 1 < n_blk) advance(c);
    }
  }
  // A run that reaches from its first prefix unit into the next one stages
  // that unit's queries too, now, while the registers are free: copied when
  // the unit starts, they would cost one memory latency per piece, each
  // waiting for the whole ring.
  bool staged2 = false;
  if (first.sp == 0) {
    stage_prefix(first, a_slot);
    if (a.aslot2 > 0 && (last.item != first.item || last.kvh != first.kvh)) {
      cs_cursor c2 = first;
      c2.j = c2.nb - 1;
      advance(c2);  // the first tile of the next unit
      if (c2.sp == 0) {
        stage_prefix(c2, a_slot2);
        staged2 = true;
      }
    }
  }
  stage_regs buf[STAGES];
#pragma unroll
  for (int u = 0; u < STAGES; ++u) issue(buf[u], u, pre[u]);

  // ---- consume side ----
  cs_cursor cs = first;
  bool cs_new = true;  // the next tile consumed is the first of a unit of the run
  int ua = 0;          // index of the current prefix unit among the run's
  // the lane's query operands of the current unit: column tile t's operand kk
  // holds dims kk * 32 + quad * 8 .. + 8 of column t * 16 + col16.  Up to
  // d = 128 they are read from the unit's LDS slot into registers once, when
  // the unit starts; at d = 256 the registers are not there, and every tile
  // reads them from the slot (q_lane[t] + kk * 32)
  constexpr bool kQRegs = D <= 128;
  bf16x8_t qf[kQRegs ? NT : 1][kQRegs ? D / 32 : 1];
  const uint16_t* q_lane[NT];
  // q4_0: -kQ4Bias times each column's query sum over group kk (the start of
  // that group's score product, which cancels the code bias)
  float kb[FMT == kFmtQ4 ? NT : 1][FMT == kFmtQ4 ? D / 32 : 1];
  int ntiles = 1, ncols = G;
  // a unit's first tile, at ring stage u: its queries into place
  auto start_unit = [&](const stage_regs& sr) __attribute__((always_inline)) {
    uint16_t* slot;
    if (cs.sp == 0) {
      slot = a_slot;
      if (ua == 1 && staged2) {
        slot = a_slot2;  // staged when the run started
        ++ua;
      } else if (ua++ > 0) {
        // a later prefix unit (rare: prefix units are long): copy its queries
        // now, piece by piece through registers, waiting for everything in
        // flight (no copy straight to LDS here: the compiler would then make
        // every LDS read of the loop wait for all loads)
        const uint16_t* qg = static_cast<const uint16_t*>(a.q);
        const int elems = cs.cnt * G * D;
        for (int e = lane * 8; e < elems; e += 64 * 8) {
          const int col = e / D, dim = e % D;
          const int m = col / G, h = col % G;
          *reinterpret_cast<uint4*>(a_slot + padded(e)) = *reinterpret_cast<const uint4*>(
              qg + (static_cast<int64_t>(cs.m0 + m) * a.n_q_heads + cs.kvh * G + h) * D + dim);
        }
      }
    } else {
      slot = b_slot;
#pragma unroll
      for (int i = 0; i < QPL; ++i)
        if ((i * 64 + lane) * 8 < G * D) {
          // (the offset is computed here, not kept from the start: registers)
          int e = (i * 64 + lane) * 8;
          asm volatile("" : "+v"(e));
          *reinterpret_cast<uint4*>(b_slot + padded(e)) = sr.q[i];
        }
    }
    ncols = cs.cnt * G;
    ntiles = cs.sp == 0 ? (ncols + 15) / 16 : 1;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      // columns past the unit's read a valid column; their results are discarded
      q_lane[t] = slot + ((t * 16 + col16) % ncols) * kQStride + quad * 8;
      if constexpr (kQRegs) {
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) qf[t][kk] = *reinterpret_cast<const bf16x8_t*>(q_lane[t] + kk * 32);
      }
      if constexpr (FMT == kFmtQ4) {
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
          const uint4 w = *reinterpret_cast<const uint4*>(q_lane[t] + kk * 32);
          const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
          float part = 0.f;
#pragma unroll
          for (int k = 0; k < 4; ++k) part += __uint_as_float(ws[k] << 16) + __uint_as_float(ws[k] & 0xffff0000u);
          kb[t][kk] = -kQ4Bias * sum_xor32(sum_xor16(part));
        }
      }
    }
  };

  f32x4_t o[NT][D / 16];
  float m_run[NT], l_lane[NT];
  auto reset = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int i = 0; i < D / 16; ++i) o[t][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      m_run[t] = -INFINITY;
      l_lane[t] = 0.f;
    }
  };
  reset();
  bool poisoned = false;
  uint64_t bad_members = 0;

  // One tile against the unit's column tiles (ntiles of NT; a suffix unit has
  // one): the same step as attend_block per column tile, written phase by
  // phase -- every column tile's score MFMAs, then the block maxima (their
  // cross-lane shuffles back to back), then per column tile the weights and
  // the value MFMAs -- so that the column tiles' dependency chains overlap
  // instead of running one after another.  Column tiles past the unit's
  // columns repeat a valid column; their results are discarded.
  auto attend_tiles = [&](kv_regs<D>& cur, int valid) __attribute__((always_inline)) {
    if (valid < 16) zero_v_tail<D>(cur, valid, quad);
    f32x4_t sc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t >= ntiles) continue;  // wave uniform
      sc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk)
        sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, cur.k[kk]),
                                                        kQRegs ? qf[kQRegs ? t : 0][kQRegs ? kk : 0]
                                                               : *reinterpret_cast<const bf16x8_t*>(q_lane[t] + kk * 32),
                                                        sc[t], 0, 0, 0);
    }
    // slots past `valid` (a partial last tile) out of the maxima and weights
    if (valid < 16) {  // wave uniform
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t >= ntiles) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (quad * 4 + i >= valid) sc[t][i] = -INFINITY;
      }
    }
    // block maxima, scaled after the reduction (the scale is positive, so the
    // maximum of the scaled scores is the scaled maximum)
    float mb[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t >= ntiles) continue;
      mb[t] = maxn_xor16(maxn(maxn3(sc[t][0], sc[t][1], sc[t][2]), sc[t][3]));
    }
    bool grow_any = false;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t >= ntiles) continue;
      mb[t] = maxn_xor32(mb[t]) * a.scale_log2;
      grow_any |= mb[t] > m_run[t] + kRescaleSlack;
    }
    // one wave-uniform branch for every column tile's rescale (rare: the
    // running maxima move by more than the slack); a column tile that did
    // not grow is scaled by 2^0 = 1
    if (__builtin_amdgcn_ballot_w64(grow_any)) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t >= ntiles) continue;
        const float m_new = mb[t] > m_run[t] + kRescaleSlack ? mb[t] : m_run[t];
        const float alpha = __builtin_amdgcn_exp2f(m_run[t] - m_new);
        l_lane[t] *= alpha;
#pragma unroll
        for (int i = 0; i < D / 16; ++i) o[t][i] *= alpha;
        m_run[t] = m_new;
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t >= ntiles) continue;
      // weights 2^(s * scale_log2 - m_run); a slot out of range has s = -inf
      // and weight 0 (m_run is finite here: the tile has a slot in range, and
      // a tile without one is a bad tile, whose result is NaN anyway)
      float pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][i], a.scale_log2, -m_run[t]));
      // bf16 weights; the denominator sums the rounded weights (as attend_block)
      const uint32_t w01 = pack_bf16x2(pv[0], pv[1]);
      const uint32_t w23 = pack_bf16x2(pv[2], pv[3]);
      l_lane[t] += (__uint_as_float(w01 << 16) + __uint_as_float(w01 & 0xffff0000u)) +
                   (__uint_as_float(w23 << 16) + __uint_as_float(w23 & 0xffff0000u));
      const s16x4_t pop = __builtin_bit_cast(s16x4_t, make_uint2(w01, w23));
#pragma unroll
      for (int pp = 0; pp < D / 32; ++pp) {
        const uint2* halves = reinterpret_cast<const uint2*>(&cur.v[pp]);
        o[t][2 * pp] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, halves[0]), pop,
                                                                 o[t][2 * pp], 0, 0, 0);
        o[t][2 * pp + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, halves[1]), pop,
                                                                     o[t][2 * pp + 1], 0, 0, 0);
      }
    }
    // the accumulators stay in the accumulation registers from tile to tile
    // (left to itself the compiler copies all of them to vector registers
    // after every tile, for the rare rescale and the end-of-run store)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < D / 16; ++i) asm volatile("" : "+a"(o[t][i]));
  };

  // The same step on a raw quantised tile: the codes as exact bf16 operands,
  // each group's score product scaled by the tile's K scale of that group and
  // slot, the V scales folded into one weight operand per group (a slot past
  // `valid` gets weight 0 by selection: its scale and codes may be anything);
  // l sums the unrounded weights, as the decode kernel's quantised step.
  auto attend_tiles_q = [&](const auto& raw, int valid) __attribute__((always_inline)) {
    kv_regs<D> cur;
    codes_block<D, FMT>(raw, cur);
    f32x4_t sc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t >= ntiles) continue;  // wave uniform
      sc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        const float b0 = FMT == kFmtQ4 ? kb[FMT == kFmtQ4 ? t : 0][FMT == kFmtQ4 ? kk : 0] : 0.f;
        const f32x4_t x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8_t, cur.k[kk]),
            kQRegs ? qf[kQRegs ? t : 0][kQRegs ? kk : 0] : *reinterpret_cast<const bf16x8_t*>(q_lane[t] + kk * 32),
            (f32x4_t{b0, b0, b0, b0}), 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[t][i] = __builtin_fmaf(scale_at<D>(raw.ks, i, kk), x[i], sc[t][i]);
      }
    }
    if (valid < 16) {  // wave uniform
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t >= ntiles) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (quad * 4 + i >= valid) sc[t][i] = -INFINITY;
      }
    }
    float mb[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t >= ntiles) continue;
      mb[t] = maxn_xor16(maxn(maxn3(sc[t][0], sc[t][1], sc[t][2]), sc[t][3]));
    }
    bool grow_any = false;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t >= ntiles) continue;
      mb[t] = maxn_xor32(mb[t]) * a.scale_log2;
      grow_any |= mb[t] > m_run[t] + kRescaleSlack;
    }
    if (__builtin_amdgcn_ballot_w64(grow_any)) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t >= ntiles) continue;
        const float m_new = mb[t] > m_run[t] + kRescaleSlack ? mb[t] : m_run[t];
        const float alpha = __builtin_amdgcn_exp2f(m_run[t] - m_new);
        l_lane[t] *= alpha;
#pragma unroll
        for (int i = 0; i < D / 16; ++i) o[t][i] *= alpha;
        m_run[t] = m_new;
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t >= ntiles) continue;
      float pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][i], a.scale_log2, -m_run[t]));
      l_lane[t] += (pv[0] + pv[1]) + (pv[2] + pv[3]);
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
        o[t][2 * pp] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, halves[0]), pop,
                                                                 o[t][2 * pp], 0, 0, 0);
        o[t][2 * pp + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, halves[1]), pop,
                                                                     o[t][2 * pp + 1], 0, 0, 0);
        if constexpr (FMT == kFmtQ4) {
          const s16x4_t nb = __builtin_bit_cast(s16x4_t, make_uint2(kQ4NegBiasPair, kQ4NegBiasPair));
          o[t][2 * pp] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(nb, pop, o[t][2 * pp], 0, 0, 0);
          o[t][2 * pp + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(nb, pop, o[t][2 * pp + 1], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < D / 16; ++i) asm volatile("" : "+a"(o[t][i]));
  };

  // writes the partial of the current unit's run and resets the state
  auto finish = [&]() __attribute__((always_inline)) {
    const int64_t unit = static_cast<int64_t>(cs.item) * Hkv + cs.kvh;
    const int64_t slot = wid + unit;  // prefix slots: < W + n_a Hkv; suffix slots from n_a Hkv on
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t >= ntiles) continue;  // wave uniform
      const float l = sum_xor32(sum_xor16(l_lane[t]));
      const int col = t * 16 + col16;
      if (col >= ncols) continue;
      // (the member index is computed here, not hoisted out of the loop as a
      // mask per column tile: those masks would take registers the ring needs)
      int member_of_col = col / G;
      asm volatile("" : "+v"(member_of_col));
      const bool bad = poisoned || ((bad_members >> member_of_col) & 1ull);
      const int64_t row = cs.sp == 0 ? slot * a.acol + col
                                     : (slot - static_cast<int64_t>(na) * Hkv) * G + col;
      float* po = (cs.sp == 0 ? a.a_o : a.b_o) + row * D;
#pragma unroll
      for (int nt = 0; nt < D / 16; ++nt)
        *reinterpret_cast<float4*>(po + nt * 16 + quad * 4) =
            bad ? make_float4(nan, nan, nan, nan) : make_float4(o[t][nt][0], o[t][nt][1], o[t][nt][2], o[t][nt][3]);
      if (quad == 0) {
        (cs.sp == 0 ? a.a_m : a.b_m)[row] = bad ? nan : m_run[t];
        (cs.sp == 0 ? a.a_l : a.b_l)[row] = bad ? nan : l;
      }
    }
    reset();
    poisoned = false;
    bad_members = 0;
  };

  int k0 = 0;
  do {
#pragma unroll
    for (int u = 0; u < STAGES; ++u) {
      const int k = k0 + u;
      if (k < n_blk) {
        if (cs_new) {
          start_unit(buf[u]);
          cs_new = false;
        }
        const bool bad = bad_ring[u];
        poisoned |= bad;
        if (cs.sp == 0)
          bad_members |= __builtin_amdgcn_ballot_w64(lane < cs.cnt && chk_ring[u] != phys_ring[u]);
        const int valid = bad ? 0 : min(16, cs.n - (cs.j0 + cs.j) * 16);
        if constexpr (FMT == kFmtBf16)
          attend_tiles(buf[u].kv, valid);
        else
          attend_tiles_q(buf[u].kv, valid);
        if (cs.j == cs.nb - 1 || k == n_blk - 1) {  // end of this unit's run
          finish();
          if (k + 1 < n_blk) {
            advance(cs);
            cs_new = true;
          }
        } else {
          advance(cs);
        }
      }
      issue(buf[u], u, entry_of(ld));
    }
    k0 += STAGES;
  } while (k0 < n_blk);
}

// One wave per (member, query head): the partials of the member's prefix unit
// (the waves whose runs cover it) and of its suffix unit, folded with
// M = max m, out = sum 2^(m - M) O / sum 2^(m - M) l.  A member the plan marked
// (prefix not covered, malformed or oversized group), or a NaN partial (a bad
// table entry, a mismatched shared entry), gives a NaN row; no keys at all, a
// zero row.
constexpr int kCsMergeBatch = 8;

template <int D>
__global__ void __launch_bounds__(256) cascade_merge_kernel(cs_args a) {
  const int lane = threadIdx.x & 63;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (item >= static_cast<int64_t>(a.n_seqs) * a.n_q_heads) return;
  const int s = static_cast<int>(item / a.n_q_heads);
  const int head = static_cast<int>(item % a.n_q_heads);
  const int G = a.n_q_heads / a.n_kv_heads;
  const int Hkv = a.n_kv_heads;
  const int kvh = head / G, hg = head % G;
  constexpr int E = (D + 63) / 64;
  uint16_t* orow = static_cast<uint16_t*>(a.out) + item * D;
  // the member's plan and its units' waves, loaded together
  const int4 mi = a.member[s];
  const int4 md = a.mdesc[static_cast<int64_t>(s) * Hkv + kvh];
  const int64_t W = a.n_waves;
  const int na = a.n_groups * a.cpg;
  const cs_split split(a.cum_parts, a.cum_cost, na + a.n_seqs, na, Hkv, a.wa, a.wb, a.wu, W);
  const int64_t wFA = md.x, wFB = md.z;
  const int64_t uA = static_cast<int64_t>(mi.y) * Hkv + kvh;
  const int64_t uB = static_cast<int64_t>(s) * Hkv + kvh;
  const int n_a = md.y;
  const int n_ent = md.y + md.w;
  const int col_a = mi.z + hg;
  // entry i: prefix wave wFA + i (i < n_a), else suffix wave wFB + i - n_a:
  // its partial row, and whether that wave wrote one (a wave without
  // partitions wrote nothing: only the unweighted split has such waves)
  auto entry_row = [&](int i, int64_t& row) -> bool {
    const bool pre = i < n_a;
    const int64_t w = pre ? wFA + i : wFB + (i - n_a);
    row = pre ? (w + uA) * a.acol + col_a : (w + uB) * G + hg;
    return split.weighted || div_nn(w * split.C, W) < div_nn((w + 1) * split.C, W);
  };
  auto entry = [&](int i, float& m, float& l, int64_t& row) {
    const bool pre = i < n_a;
    m = -INFINITY;
    l = 0.f;
    if (!entry_row(i, row)) {
      row = 0;
      return;
    }
    m = (pre ? a.a_m : a.b_m)[row];
    l = (pre ? a.a_l : a.b_l)[row];
  };
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  float M = -INFINITY, L = 0.f;
  bool nan_seen = mi.x < 0;
  // weighted rows of the entries [i0, i0 + cnt), whose weights and rows lanes
  // 0 .. cnt-1 hold: loaded kCsMergeBatch at a time with no branch between the
  // loads, so a batch waits out one memory latency
  auto accumulate = [&](int i0, int cnt, float w, int64_t row) {
    const int row_lo = static_cast<int>(row & 0xffffffff), row_hi = static_cast<int>(row >> 32);
    for (int k0 = 0; k0 < cnt; k0 += kCsMergeBatch) {
      float v[kCsMergeBatch][E];
#pragma unroll
      for (int k = 0; k < kCsMergeBatch; ++k) {
        const int kk = min(k0 + k, cnt - 1);  // past the end: a repeat, weight 0 below
        const int64_t rk = (static_cast<int64_t>(__shfl(row_hi, kk)) << 32) | static_cast<uint32_t>(__shfl(row_lo, kk));
        const float* src = (i0 + kk < n_a ? a.a_o : a.b_o) + rk * D;
#pragma unroll
        for (int e = 0; e < E; ++e) v[k][e] = lane + 64 * e < D ? src[lane + 64 * e] : 0.f;
      }
#pragma unroll
      for (int k = 0; k < kCsMergeBatch; ++k) {
        const float wk = k0 + k < cnt ? __shfl(w, k0 + k) : 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = wk == 0.f ? acc[e] : __builtin_fmaf(wk, v[k][e], acc[e]);
      }
    }
  };
  if (n_ent > 0 && n_ent <= kCsMergeBatch) {
    // the usual case: lane i loads entry i's (m, l) and every lane its slice
    // of every entry's row, all at once (one memory latency)
    float m, l;
    int64_t row;
    entry(lane < n_ent ? lane : 0, m, l, row);
    if (lane >= n_ent) {
      m = -INFINITY;
      l = 0.f;
    }
    const int row_lo = static_cast<int>(row & 0xffffffff), row_hi = static_cast<int>(row >> 32);
    float v[kCsMergeBatch][E];
#pragma unroll
    for (int k = 0; k < kCsMergeBatch; ++k) {
      const int kk = min(k, n_ent - 1);  // past the end: a repeat, weight 0 below
      const int64_t rk = (static_cast<int64_t>(__shfl(row_hi, kk)) << 32) | static_cast<uint32_t>(__shfl(row_lo, kk));
      const float* src = (kk < n_a ? a.a_o : a.b_o) + rk * D;
#pragma unroll
      for (int e = 0; e < E; ++e) v[k][e] = lane + 64 * e < D ? src[lane + 64 * e] : 0.f;
    }
    nan_seen |= __builtin_amdgcn_ballot_w64(m != m) != 0;
    M = wave_max(m != m ? -INFINITY : m);
    const float w = (m == -INFINITY || m != m) ? 0.f : exp2f(m - M);
    L = wave_sum(w == 0.f ? 0.f : w * l);
#pragma unroll
    for (int k = 0; k < kCsMergeBatch; ++k) {
      const float wk = k < n_ent ? __shfl(w, k) : 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = wk == 0.f ? acc[e] : __builtin_fmaf(wk, v[k][e], acc[e]);
    }
  } else if (n_ent > 0 && n_ent <= 64) {
    // every lane resolves one entry once
    float m, l;
    int64_t row;
    entry(lane < n_ent ? lane : 0, m, l, row);
    if (lane >= n_ent) {
      m = -INFINITY;
      l = 0.f;
    }
    nan_seen |= __builtin_amdgcn_ballot_w64(m != m) != 0;
    M = wave_max(m != m ? -INFINITY : m);
    const float w = (m == -INFINITY || m != m) ? 0.f : exp2f(m - M);
    L = wave_sum(w == 0.f ? 0.f : w * l);
    accumulate(0, n_ent, w, row);
  } else if (n_ent > 64) {
    for (int i0 = 0; i0 < n_ent; i0 += 64) {
      float m = -INFINITY, l = 0.f;
      int64_t row = 0;
      if (i0 + lane < n_ent) entry(i0 + lane, m, l, row);
      nan_seen |= __builtin_amdgcn_ballot_w64(m != m) != 0;
      M = fmaxf(M, wave_max(m != m ? -INFINITY : m));
    }
    for (int i0 = 0; i0 < n_ent; i0 += 64) {
      float m = -INFINITY, l = 0.f;
      int64_t row = 0;
      if (i0 + lane < n_ent) entry(i0 + lane, m, l, row);
      const float w = (m == -INFINITY || m != m) ? 0.f : exp2f(m - M);
      L += wave_sum(w == 0.f ? 0.f : w * l);
      accumulate(i0, min(64, n_ent - i0), w, row);
    }
  }
  const bool empty = M == -INFINITY && !nan_seen;  // no key at all
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (lane + 64 * e < D)
      orow[lane + 64 * e] = nan_seen ? static_cast<uint16_t>(0x7fc0) : (empty ? 0 : f32_to_bf16(acc[e] / L));
}

// ---- host side ---------------------------------------------------------------

struct cs_plan {
  int nt, acol, mc, cpg, na, aslot, aslot2, bslot, part_blocks, wa, wb, wu;
  int64_t waves;
  uint64_t lds;
  uint64_t a_m, a_l, a_o, b_m, b_l, b_o, cum_parts, cum_cost, member, mdesc, total;  // workspace offsets
  float scale;
};

kv_status cs_resolve(const kv_pool* pool, int n_seqs, int n_groups, int max_group, int num_q_heads, int max_blocks,
                     const kv_attention_options* opts, cs_plan& p) {
  if (!pool) return fail(KV_ERR_INVALID, "pool is NULL");
  const kv_pool_config& c = pool->cfg;
  if (num_q_heads <= 0 || num_q_heads % c.num_kv_heads != 0)
    return fail(KV_ERR_INVALID, "num_q_heads must be a positive multiple of num_kv_heads");
  const int G = num_q_heads / c.num_kv_heads;
  kv_attention_options o{0.f, 0, KV_KERNEL_AUTO, nullptr};
  if (opts) o = *opts;
  if (o.kernel != KV_KERNEL_AUTO && o.kernel != KV_KERNEL_MFMA && o.kernel != KV_KERNEL_GENERIC)
    return fail(KV_ERR_INVALID, "unknown kernel selector");
  if (!mfma_supported(c, G) || o.kernel == KV_KERNEL_GENERIC)
    return fail(KV_ERR_UNSUPPORTED, "the cascade decode needs a bf16, q8_0 or q4_0 pool with B = 16, d in {64, 128, "
                                    "256}, G <= 16 and the matrix-core kernel");
  if (n_seqs < 1 || max_blocks <= 0) return fail(KV_ERR_INVALID, "n_seqs and max_blocks_per_seq must be positive");
  if (n_groups < 1 || n_groups > n_seqs || max_group < 1)
    return fail(KV_ERR_INVALID, "need 1 <= n_groups <= n_seqs and max_group >= 1");
  if (o.partition_tokens < 0 || o.partition_tokens % 16 != 0)
    return fail(KV_ERR_INVALID, "partition_tokens must be 0 or a positive multiple of the block size");
  if (!(o.scale >= 0.f) || std::isinf(o.scale)) return fail(KV_ERR_INVALID, "scale must be finite and >= 0");
  p.scale = o.scale > 0.f ? o.scale : 1.f / std::sqrt(static_cast<float>(c.head_dim));
  p.part_blocks = o.partition_tokens ? o.partition_tokens / 16 : 1;
  p.nt = cs_tiles_rt(c.head_dim, c.dtype);
  p.acol = 16 * p.nt;
  p.waves = static_cast<int64_t>(kCsWaves) * device_cus();
  // LDS: the plan, then per wave a prefix slot of mc members' queries and a
  // ring of cs_stages + 1 suffix slots; mc is as many members as the column
  // tiles hold, fewer where the slots would not fit
  const int D = c.head_dim;
  // slots hold columns D + 8 elements apart (see the kernel), rounded to 16 bytes
  const int64_t stride = D + 8;
  p.bslot = static_cast<int>(G * stride);
  const int qb = 1;  // one suffix slot per wave
  const int64_t lds_max = static_cast<int64_t>(max_lds_per_block()) - 256;  // the kernel's own static LDS
  int mc = p.acol / G;
  const int nt_cap = std::min(max_group, n_seqs);
  for (; mc >= 1; --mc) {
    const int na = n_groups * ((nt_cap + mc - 1) / mc);
    const int64_t lds = static_cast<int64_t>(cs_lds_ints(na + n_seqs, n_seqs, n_groups)) * 4 +
                        static_cast<int64_t>(kCsWaves) * (mc * G * stride + qb * p.bslot) * 2;
    if (lds <= lds_max) break;
  }
  if (mc < 1)
    return fail(KV_ERR_UNSUPPORTED, "too many sequences or prefix chunks for the cascade decode's plan in LDS "
                                    "(pass the largest group size as max_group)");
  p.mc = mc;
  p.aslot = static_cast<int>(mc * G * stride);
  // a second prefix slot per wave where the LDS holds it (a run reaching into
  // a second prefix unit stages its queries at the start)
  const int64_t lds_one = static_cast<int64_t>(cs_lds_ints(n_groups * ((nt_cap + mc - 1) / mc) + n_seqs, n_seqs, n_groups)) * 4 +
                          static_cast<int64_t>(kCsWaves) * (p.aslot + qb * p.bslot) * 2;
  p.aslot2 = lds_one + static_cast<int64_t>(kCsWaves) * p.aslot * 2 <= lds_max ? p.aslot : 0;
  // work-split weights, in quarters of a suffix tile (one column tile): a
  // tile attended by a full chunk's ct column tiles costs about 3 + ct, the
  // start of a unit about 6
  p.wa = 3 + (mc * G + 15) / 16;
  p.wb = 4;
  p.wu = 6;
  p.cpg = (nt_cap + p.mc - 1) / p.mc;
  p.na = n_groups * p.cpg;
  // the plan's per-kv-head sums (tiles, partitions, costs) are 32-bit
  if (static_cast<int64_t>(p.na + n_seqs) * (static_cast<int64_t>(max_blocks) * std::max(p.wa, p.wb) + p.wu) >
      std::numeric_limits<int32_t>::max())
    return fail(KV_ERR_UNSUPPORTED, "too many sequences x blocks for the cascade decode's plan");
  p.lds = static_cast<uint64_t>(cs_lds_ints(p.na + n_seqs, n_seqs, n_groups)) * 4 +
          static_cast<uint64_t>(kCsWaves) * (p.aslot + p.aslot2 + qb * p.bslot) * 2;
  const uint64_t Hkv = c.num_kv_heads;
  const uint64_t a_rows = (static_cast<uint64_t>(p.waves) + p.na * Hkv) * p.acol;
  const uint64_t b_rows = (static_cast<uint64_t>(p.waves) + n_seqs * Hkv) * G;
  uint64_t at = 0;
  auto take = [&](uint64_t bytes) {
    const uint64_t o = at;
    at += up256(bytes);
    return o;
  };
  p.a_m = take(a_rows * 4);
  p.a_l = take(a_rows * 4);
  p.a_o = take(a_rows * c.head_dim * 4);
  p.b_m = take(b_rows * 4);
  p.b_l = take(b_rows * 4);
  p.b_o = take(b_rows * c.head_dim * 4);
  p.cum_parts = take((p.na + n_seqs + 1) * 4ull);
  p.cum_cost = take((p.na + n_seqs + 1) * 4ull);
  p.member = take(n_seqs * 16ull);
  p.mdesc = take(n_seqs * Hkv * 16ull);
  p.total = at;
  return KV_OK;
}

template <int D, int QPL, int FMT>
hipError_t cs_launch_q(const cs_args& a, const cs_plan& p, hipStream_t st, const call_events& ev) {
  return launch_timed(attn_cascade_kernel<D, cs_stages(D, QPL), QPL, FMT>, dim3(static_cast<unsigned>(p.waves / kCsWaves)),
                      dim3(kCsWaves * 64), static_cast<uint32_t>(p.lds), st, ev.start, ev.kernel_stop, a);
}

template <int D, int FMT>
hipError_t cs_launch(const cs_args& a, const cs_plan& p, hipStream_t st, const call_events& ev) {
  // 16-byte pieces per lane of a suffix unit's G x D queries
  const int qpl = (a.n_q_heads / a.n_kv_heads * D + 511) / 512;
  hipError_t e;
  // (G <= 16: at most 16 D / 512 pieces)
  if (qpl <= 1) e = cs_launch_q<D, 1, FMT>(a, p, st, ev);
  else if (qpl <= 2 || D == 64) e = cs_launch_q<D, 2, FMT>(a, p, st, ev);
  else if (qpl <= 4 || D == 128) e = cs_launch_q<D, std::min(4, 16 * D / 512), FMT>(a, p, st, ev);
  else e = cs_launch_q<D, 16 * D / 512, FMT>(a, p, st, ev);
  if (e != hipSuccess) return e;
  const int64_t items = static_cast<int64_t>(a.n_seqs) * a.n_q_heads;
  return launch_timed(cascade_merge_kernel<D>, dim3(static_cast<unsigned>((items + 3) / 4)), dim3(256), 0u, st,
                      nullptr, ev.stop, a);
}

template <int D>
hipError_t cs_dispatch(int32_t dtype, const cs_args& a, const cs_plan& p, hipStream_t st, const call_events& ev) {
  if (dtype == KV_Q8_0) return cs_launch<D, kFmtQ8>(a, p, st, ev);
  if (dtype == KV_Q4_0) return cs_launch<D, kFmtQ4>(a, p, st, ev);
  return cs_launch<D, kFmtBf16>(a, p, st, ev);
}

}  // namespace
}  // namespace pagedkv

using namespace pagedkv;

extern "C" {

uint64_t paged_attention_cascade_workspace_bytes(kv_pool* pool, int32_t n_seqs, int32_t n_groups, int32_t max_group,
                                                 int32_t num_q_heads, int32_t max_blocks_per_seq,
                                                 const kv_attention_options* opts) {
  if (!pool || n_seqs <= 0) return 0;
  cs_plan p;
  if (cs_resolve(pool, n_seqs, n_groups, max_group, num_q_heads, max_blocks_per_seq, opts, p) != KV_OK) return 0;
  return p.total;
}

kv_status paged_attention_decode_cascade(kv_pool* pool, int32_t layer, const void* q, void* out,
                                         const int32_t* d_block_tables, const int32_t* d_context_lens,
                                         int32_t n_seqs, int32_t max_blocks_per_seq, int32_t num_q_heads,
                                         const int32_t* d_group_start, const int32_t* d_shared_blocks,
                                         int32_t n_groups, int32_t max_group, const kv_attention_options* opts,
                                         void* d_workspace, uint64_t workspace_bytes, void* hip_stream) {
  if (!pool) return fail(KV_ERR_INVALID, "pool is NULL");
  const kv_pool_config& c = pool->cfg;
  if (layer < 0 || layer >= c.num_layers) return fail(KV_ERR_INVALID, "layer out of range");
  if (n_seqs == 0) return KV_OK;
  cs_plan p;
  if (kv_status s = cs_resolve(pool, n_seqs, n_groups, max_group, num_q_heads, max_blocks_per_seq, opts, p)) return s;
  if (!q || !out || !d_block_tables || !d_context_lens || !d_group_start || !d_shared_blocks || !pool->k_cache ||
      !pool->v_cache)
    return fail(KV_ERR_INVALID, "NULL device pointer");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out)) & 15)
    return fail(KV_ERR_INVALID, "q and out must be 16-byte aligned");
  if (!d_workspace || workspace_bytes < p.total)
    return fail(KV_ERR_INVALID, "workspace too small: need " + std::to_string(p.total) + " bytes");
  if (reinterpret_cast<uintptr_t>(d_workspace) & 255) return fail(KV_ERR_INVALID, "workspace must be 256-byte aligned");
  char* ws = static_cast<char*>(d_workspace);
  const int64_t layer_off = static_cast<int64_t>(layer) * c.num_blocks * c.num_kv_heads * tile_bytes(c);
  cs_args a{};
  a.q = q;
  a.out = out;
  a.k_layer = static_cast<const char*>(pool->k_cache) + layer_off;
  a.v_layer = static_cast<const char*>(pool->v_cache) + layer_off;
  a.tables = d_block_tables;
  a.ctx_lens = d_context_lens;
  a.group_start = d_group_start;
  a.shared = d_shared_blocks;
  a.a_m = reinterpret_cast<float*>(ws + p.a_m);
  a.a_l = reinterpret_cast<float*>(ws + p.a_l);
  a.a_o = reinterpret_cast<float*>(ws + p.a_o);
  a.b_m = reinterpret_cast<float*>(ws + p.b_m);
  a.b_l = reinterpret_cast<float*>(ws + p.b_l);
  a.b_o = reinterpret_cast<float*>(ws + p.b_o);
  a.cum_parts = reinterpret_cast<int32_t*>(ws + p.cum_parts);
  a.cum_cost = reinterpret_cast<int32_t*>(ws + p.cum_cost);
  a.member = reinterpret_cast<int4*>(ws + p.member);
  a.mdesc = reinterpret_cast<int4*>(ws + p.mdesc);
  a.n_seqs = n_seqs;
  a.n_groups = n_groups;
  a.cpg = p.cpg;
  a.mc = p.mc;
  a.max_group = max_group;
  a.max_blocks = max_blocks_per_seq;
  a.n_q_heads = num_q_heads;
  a.n_kv_heads = c.num_kv_heads;
  a.num_blocks = c.num_blocks;
  a.part_blocks = p.part_blocks;
  a.n_waves = static_cast<int>(p.waves);
  a.acol = p.acol;
  a.wa = p.wa;
  a.wb = p.wb;
  a.wu = p.wu;
  a.aslot = p.aslot;
  a.aslot2 = p.aslot2;
  a.bslot = p.bslot;
  a.scale_log2 = p.scale * kLog2e;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const call_events ev = events_of(opts);
  hipError_t e;
  switch (c.head_dim) {
    case 64: e = cs_dispatch<64>(c.dtype, a, p, st, ev); break;
    case 128: e = cs_dispatch<128>(c.dtype, a, p, st, ev); break;
    default: e = cs_dispatch<256>(c.dtype, a, p, st, ev); break;
  }
  return hip_check(e, "cascade decode launch");
}

}  // extern "C"
