// Host block manager of the paged KV cache: free list, reference counts,
// block tables, append with copy-on-write, fork, deferred release.
//
// Sources (by page title):
//   [BT]  "PagedAttention 的块表与碎片控制" (block tables and fragmentation):
//         §03 translation j = t / B, r = t mod B; §04 grow by one block when the
//         last one is full; §05 FIFO free list, error on an empty list;
//         §08 reference counts and copy-on-write; §10 reserve a step's blocks
//         atomically; §13 conservation N_free + N_allocated = N_total.
//   [KVM] "KV 缓存管理" (KV cache management), "Zero-copy branching via
//         copy-on-write": fork copies the table and increments each block's
//         count; a write into a block with count > 1 first takes a private copy;
//         release decrements and returns blocks reaching zero.
//   [INF] "第 8 章 推理优化", §8.3.2: a block is reusable only when no
//         reference remains and submitted device work no longer reads it.
//   [KVM] asynchronous paged swap (Figure 11 and its three migration steps):
//         frames of a pinned host pool, a block table whose entries carry
//         their residency, device blocks returned once the copy is done.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstring>
#include <numeric>
#include <string>

#include "pool_internal.h"

namespace pagedkv {

static thread_local std::string g_last_error;

kv_status fail(kv_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

static kv_status ok() {
  g_last_error.clear();
  return KV_OK;
}

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

static kv_status validate_config(const kv_pool_config* c) {
  if (!c) return fail(KV_ERR_INVALID, "config is NULL");
  if (c->num_layers <= 0 || c->num_blocks <= 0 || c->block_size <= 0 || c->num_kv_heads <= 0)
    return fail(KV_ERR_INVALID, "num_layers, num_blocks, block_size and num_kv_heads must be positive");
  if (c->head_dim <= 0 || c->head_dim % 32 != 0 || c->head_dim > 256)
    return fail(KV_ERR_INVALID, "head_dim must be a positive multiple of 32, at most 256");
  if (c->dtype != KV_F32 && c->dtype != KV_BF16 && c->dtype != KV_Q8_0 && c->dtype != KV_Q4_0)
    return fail(KV_ERR_INVALID, "dtype must be KV_F32, KV_BF16, KV_Q8_0 or KV_Q4_0");
  if (pagedkv::is_quantized(c->dtype) &&
      (c->block_size != 16 || (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256)))
    return fail(KV_ERR_UNSUPPORTED, "a quantised pool needs B = 16 and head_dim 64, 128 or 256");
  if (static_cast<int64_t>(c->num_blocks) * c->block_size > INT64_C(1) << 40)
    return fail(KV_ERR_INVALID, "pool too large");
  return KV_OK;
}

// Moves the blocks of ready pending groups to the back of the free list, in
// release order; groups still waiting keep their place.
static void reclaim_ready(kv_pool* p, bool wait) {
  std::deque<kv_pending_group> waiting;
  for (auto& g : p->pending) {
    if (!g.ready && g.event) {
      hipEvent_t ev = static_cast<hipEvent_t>(g.event);
      if ((wait ? hipEventSynchronize(ev) : hipEventQuery(ev)) == hipSuccess) g.ready = true;
    }
    if (g.ready) {
      for (int32_t b : g.blocks) p->free_list.push_back(b);
      for (int32_t f : g.frames) p->host_free.push_back(f);
      p->n_pending -= static_cast<int32_t>(g.blocks.size());
      p->n_host_pending -= static_cast<int32_t>(g.frames.size());
      if (g.event) (void)hipEventDestroy(static_cast<hipEvent_t>(g.event));
    } else {
      waiting.push_back(std::move(g));
    }
  }
  p->pending.swap(waiting);
}

// Refuses a sequence that has host-resident entries.
static kv_status resident(const kv_seq_state& s, int64_t seq) {
  if (s.n_host > 0) return fail(KV_ERR_INVALID, "sequence " + std::to_string(seq) + " is swapped out");
  return KV_OK;
}

// Event recorded on a stream, for a pending group.
static kv_status record_event(void* hip_stream, void** out) {
  hipEvent_t ev = nullptr;
  hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
  if (e != hipSuccess) return fail(KV_ERR_HIP, std::string("hipEventCreateWithFlags: ") + hipGetErrorString(e));
  e = hipEventRecord(ev, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) {
    (void)hipEventDestroy(ev);
    return fail(KV_ERR_HIP, std::string("hipEventRecord: ") + hipGetErrorString(e));
  }
  *out = ev;
  return KV_OK;
}

}  // namespace pagedkv

using namespace pagedkv;

extern "C" {

const char* kv_last_error(void) { return g_last_error.c_str(); }

kv_status kv_pool_required_bytes(const kv_pool_config* cfg, uint64_t* k_bytes, uint64_t* v_bytes) {
  if (kv_status st = validate_config(cfg)) return st;
  if (!k_bytes || !v_bytes) return fail(KV_ERR_INVALID, "output pointer is NULL");
  uint64_t b = static_cast<uint64_t>(pool_bytes(*cfg));
  *k_bytes = b;
  *v_bytes = b;
  return ok();
}

kv_status kv_pool_create(const kv_pool_config* cfg, void* k_cache, void* v_cache,
                         const int32_t* initial_free_order, kv_pool** out) {
  if (kv_status st = validate_config(cfg)) return st;
  if (!out) return fail(KV_ERR_INVALID, "out is NULL");
  const int32_t n = cfg->num_blocks;
  std::vector<int32_t> order(n);
  if (initial_free_order) {
    std::vector<char> seen(n, 0);
    for (int32_t i = 0; i < n; ++i) {
      int32_t b = initial_free_order[i];
      if (b < 0 || b >= n || seen[b]) return fail(KV_ERR_INVALID, "initial_free_order is not a permutation of 0..N-1");
      seen[b] = 1;
      order[i] = b;
    }
  } else {
    std::iota(order.begin(), order.end(), 0);
  }
  kv_pool* p = new kv_pool();
  p->cfg = *cfg;
  p->k_cache = k_cache;
  p->v_cache = v_cache;
  p->free_list.assign(order.begin(), order.end());
  p->ref.assign(n, 0);
  *out = p;
  return ok();
}

void kv_pool_destroy(kv_pool* p) {
  if (!p) return;
  for (auto& g : p->pending)
    if (g.event) (void)hipEventDestroy(static_cast<hipEvent_t>(g.event));
  prefix_destroy(p);
  delete p;
}

kv_status kv_seq_add(kv_pool* p, int64_t seq_id) {
  if (!p) return fail(KV_ERR_INVALID, "pool is NULL");
  if (p->seqs.count(seq_id)) return fail(KV_ERR_INVALID, "sequence " + std::to_string(seq_id) + " already exists");
  p->seqs.emplace(seq_id, kv_seq_state{});
  return ok();
}

kv_status kv_seq_fork(kv_pool* p, int64_t parent, int64_t child) {
  if (!p) return fail(KV_ERR_INVALID, "pool is NULL");
  auto it = p->seqs.find(parent);
  if (it == p->seqs.end()) return fail(KV_ERR_INVALID, "unknown parent " + std::to_string(parent));
  if (p->seqs.count(child)) return fail(KV_ERR_INVALID, "sequence " + std::to_string(child) + " already exists");
  if (kv_status r = resident(it->second, parent)) return r;
  kv_seq_state st = it->second;  // table copy
  for (int32_t b : st.table) p->ref[b] += 1;
  p->seqs.emplace(child, std::move(st));
  return ok();
}

kv_status kv_append_slots(kv_pool* p, int32_t n, const int64_t* seq_ids, const int32_t* n_new,
                          int64_t* slot_mapping_out, int64_t slot_capacity,
                          int64_t* cow_pairs_out, int32_t cow_capacity, int32_t* n_cow_out) {
  if (!p) return fail(KV_ERR_INVALID, "pool is NULL");
  if (n < 0) return fail(KV_ERR_INVALID, "n < 0");
  if (n > 0 && (!seq_ids || !n_new)) return fail(KV_ERR_INVALID, "seq_ids or n_new is NULL");
  if (!n_cow_out) return fail(KV_ERR_INVALID, "n_cow_out is NULL");
  int64_t total = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (n_new[i] < 0) return fail(KV_ERR_INVALID, "negative token count");
    auto it = p->seqs.find(seq_ids[i]);
    if (it == p->seqs.end()) return fail(KV_ERR_INVALID, "unknown sequence " + std::to_string(seq_ids[i]));
    if (kv_status r = resident(it->second, seq_ids[i])) return r;
    total += n_new[i];
  }
  if (total > slot_capacity) return fail(KV_ERR_INVALID, "slot_mapping_out capacity too small");
  if (total > 0 && !slot_mapping_out) return fail(KV_ERR_INVALID, "slot_mapping_out is NULL");
  if (n > 0 && cow_capacity < n) return fail(KV_ERR_INVALID, "cow_capacity must be at least n");
  if (n > 0 && !cow_pairs_out) return fail(KV_ERR_INVALID, "cow_pairs_out is NULL");

  reclaim_ready(p, false);

  const int32_t B = p->cfg.block_size;
  struct undo_t {
    kv_seq_state* seq;
    int32_t old_len;
    size_t old_size;
    int32_t cow_index;
    int32_t cow_old;
  };
  std::vector<undo_t> undo;
  undo.reserve(n);
  std::vector<int32_t> popped;
  int32_t n_cow = 0;
  int64_t at = 0;
  bool oom = false;

  for (int32_t i = 0; i < n && !oom; ++i) {
    kv_seq_state& s = p->seqs[seq_ids[i]];
    undo.push_back({&s, s.length, s.table.size(), -1, -1});
    for (int32_t c = 0; c < n_new[i]; ++c) {
      const int32_t j = s.length / B;
      const int32_t r = s.length % B;
      if (j == static_cast<int32_t>(s.table.size())) {
        if (p->free_list.empty()) { oom = true; break; }
        int32_t b = p->free_list.front();
        p->free_list.pop_front();
        popped.push_back(b);
        p->ref[b] = 1;
        s.table.push_back(b);
      } else if (p->ref[s.table[j]] > 1) {
        if (p->free_list.empty()) { oom = true; break; }
        int32_t old = s.table[j];
        int32_t b = p->free_list.front();
        p->free_list.pop_front();
        popped.push_back(b);
        p->ref[b] = 1;
        p->ref[old] -= 1;
        s.table[j] = b;
        undo.back().cow_index = j;
        undo.back().cow_old = old;
        cow_pairs_out[2 * n_cow] = old;
        cow_pairs_out[2 * n_cow + 1] = b;
        ++n_cow;
      }
      slot_mapping_out[at++] = static_cast<int64_t>(s.table[j]) * B + r;
      s.length += 1;
    }
  }

  if (oom) {
    for (auto u = undo.rbegin(); u != undo.rend(); ++u) {
      if (u->cow_index >= 0) {
        u->seq->table[u->cow_index] = u->cow_old;
        p->ref[u->cow_old] += 1;
      }
      u->seq->table.resize(u->old_size);
      u->seq->length = u->old_len;
    }
    for (auto b = popped.rbegin(); b != popped.rend(); ++b) {
      p->ref[*b] = 0;
      p->free_list.push_front(*b);
    }
    *n_cow_out = 0;
    return fail(KV_ERR_OOM, "no free KV block: the batch needs more blocks than the free list holds ("
                                + std::to_string(p->free_list.size()) + " free, "
                                + std::to_string(p->n_pending) + " pending release)");
  }
  *n_cow_out = n_cow;
  return ok();
}

kv_status kv_get_block_tables(const kv_pool* p, int32_t n, const int64_t* seq_ids, int32_t max_blocks,
                              int32_t* tables_out, int32_t* context_lens_out) {
  if (!p) return fail(KV_ERR_INVALID, "pool is NULL");
  if (n < 0 || max_blocks < 0) return fail(KV_ERR_INVALID, "negative size");
  if (n > 0 && (!seq_ids || !context_lens_out || (max_blocks > 0 && !tables_out)))
    return fail(KV_ERR_INVALID, "NULL argument");
  for (int32_t i = 0; i < n; ++i) {
    auto it = p->seqs.find(seq_ids[i]);
    if (it == p->seqs.end()) return fail(KV_ERR_INVALID, "unknown sequence " + std::to_string(seq_ids[i]));
    if (kv_status r = resident(it->second, seq_ids[i])) return r;
    if (static_cast<int64_t>(it->second.table.size()) > max_blocks)
      return fail(KV_ERR_INVALID, "block table of sequence " + std::to_string(seq_ids[i]) + " is longer than max_blocks");
  }
  for (int32_t i = 0; i < n; ++i) {
    const kv_seq_state& s = p->seqs.at(seq_ids[i]);
    int32_t* row = tables_out + static_cast<int64_t>(i) * max_blocks;
    std::copy(s.table.begin(), s.table.end(), row);
    std::fill(row + s.table.size(), row + max_blocks, -1);
    context_lens_out[i] = s.length;
  }
  return ok();
}

kv_status kv_pool_get_config(const kv_pool* p, kv_pool_config* out) {
  if (!p || !out) return fail(KV_ERR_INVALID, "NULL argument");
  *out = p->cfg;
  return ok();
}

kv_status kv_seq_info(const kv_pool* p, int64_t seq_id, int32_t* length, int32_t* num_blocks) {
  if (!p) return fail(KV_ERR_INVALID, "pool is NULL");
  auto it = p->seqs.find(seq_id);
  if (it == p->seqs.end()) return fail(KV_ERR_INVALID, "unknown sequence " + std::to_string(seq_id));
  if (length) *length = it->second.length;
  if (num_blocks) *num_blocks = static_cast<int32_t>(it->second.table.size());
  return ok();
}

static kv_status release_common(kv_pool* p, int64_t seq_id, void* event, uint64_t fence, bool immediate) {
  auto it = p->seqs.find(seq_id);
  kv_pending_group g;
  g.event = event;
  g.fence = fence;
  const kv_seq_state& s = it->second;
  for (size_t j = 0; j < s.table.size(); ++j) {
    if (s.n_host > 0 && s.host[j] >= 0) {  // host-resident entry: its frame goes back
      g.frames.push_back(s.host[j]);
      continue;
    }
    const int32_t b = s.table[j];
    p->ref[b] -= 1;
    if (p->ref[b] == 0) g.blocks.push_back(b);
  }
  p->seqs.erase(it);
  prefix_on_release(p, seq_id);
  if (immediate) {
    for (int32_t b : g.blocks) p->free_list.push_back(b);
    for (int32_t f : g.frames) p->host_free.push_back(f);
    if (event) (void)hipEventDestroy(static_cast<hipEvent_t>(event));
    return ok();
  }
  p->n_pending += static_cast<int32_t>(g.blocks.size());
  p->n_host_pending += static_cast<int32_t>(g.frames.size());
  p->pending.push_back(std::move(g));
  return ok();
}

kv_status kv_seq_release(kv_pool* p, int64_t seq_id, void* hip_stream) {
  if (!p) return fail(KV_ERR_INVALID, "pool is NULL");
  if (!p->seqs.count(seq_id)) return fail(KV_ERR_INVALID, "unknown sequence " + std::to_string(seq_id));
  hipEvent_t ev = nullptr;
  hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
  if (e != hipSuccess) return fail(KV_ERR_HIP, std::string("hipEventCreateWithFlags: ") + hipGetErrorString(e));
  e = hipEventRecord(ev, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) {
    (void)hipEventDestroy(ev);
    return fail(KV_ERR_HIP, std::string("hipEventRecord: ") + hipGetErrorString(e));
  }
  return release_common(p, seq_id, ev, 0, false);
}

kv_status kv_seq_release_fenced(kv_pool* p, int64_t seq_id, uint64_t fence) {
  if (!p) return fail(KV_ERR_INVALID, "pool is NULL");
  if (!p->seqs.count(seq_id)) return fail(KV_ERR_INVALID, "unknown sequence " + std::to_string(seq_id));
  return release_common(p, seq_id, nullptr, fence, fence == 0);
}

kv_status kv_pool_retire(kv_pool* p, uint64_t completed_fence) {
  if (!p) return fail(KV_ERR_INVALID, "pool is NULL");
  for (auto& g : p->pending)
    if (!g.event && g.fence <= completed_fence) g.ready = true;
  reclaim_ready(p, false);
  return ok();
}

kv_status kv_pool_reclaim(kv_pool* p, int32_t wait) {
  if (!p) return fail(KV_ERR_INVALID, "pool is NULL");
  reclaim_ready(p, wait != 0);
  return ok();
}

kv_status kv_pool_stats(const kv_pool* p, kv_pool_stats_t* out) {
  if (!p || !out) return fail(KV_ERR_INVALID, "NULL argument");
  kv_pool_stats_t s{};
  s.n_free = static_cast<int32_t>(p->free_list.size());
  for (int32_t r : p->ref) {
    if (r > 0) ++s.n_allocated;
    if (r > 1) ++s.n_shared;
  }
  s.n_pending = p->n_pending;
  s.n_seqs = static_cast<int32_t>(p->seqs.size());
  for (const auto& kv : p->seqs) {
    s.n_tokens += kv.second.length;
    s.n_table_refs += static_cast<int64_t>(kv.second.table.size());
  }
  *out = s;
  return ok();
}

kv_status kv_shared_prefix_plan(const kv_pool* p, int32_t n, const int64_t* seq_ids, int32_t* group_start,
                                int32_t* shared_blocks, int32_t* n_groups) {
  if (!p || !n_groups || (n > 0 && (!seq_ids || !group_start || !shared_blocks)))
    return fail(KV_ERR_INVALID, "NULL argument");
  if (n < 0) return fail(KV_ERR_INVALID, "n < 0");
  std::vector<const kv_seq_state*> s(n);
  for (int32_t i = 0; i < n; ++i) {
    auto it = p->seqs.find(seq_ids[i]);
    if (it == p->seqs.end()) return fail(KV_ERR_INVALID, "unknown sequence " + std::to_string(seq_ids[i]));
    if (kv_status r = resident(it->second, seq_ids[i])) return r;
    s[i] = &it->second;
  }
  const int32_t B = p->cfg.block_size;
  // leading blocks of b that equal a's and are completely filled in both
  auto common = [&](const kv_seq_state* a, const kv_seq_state* b) {
    const int32_t lim = std::min(a->length, b->length) / B;
    int32_t j = 0;
    while (j < lim && a->table[j] == b->table[j]) ++j;
    return j;
  };
  int32_t g = 0;
  for (int32_t i = 0; i < n;) {
    int32_t shared = 0, k = i + 1;
    while (k < n) {
      const int32_t c = common(s[i], s[k]);
      if (c < 1) break;
      shared = (k == i + 1) ? c : std::min(shared, c);
      ++k;
    }
    group_start[g] = i;
    shared_blocks[g] = shared;
    ++g;
    i = k;
  }
  group_start[g] = n;
  *n_groups = g;
  return ok();
}

kv_status kv_pool_free_list(const kv_pool* p, int32_t cap, int32_t* out, int32_t* n_out) {
  if (!p || !n_out) return fail(KV_ERR_INVALID, "NULL argument");
  const int32_t n = static_cast<int32_t>(p->free_list.size());
  *n_out = n;
  if (cap < n || (n > 0 && !out)) return fail(KV_ERR_INVALID, "capacity too small");
  std::copy(p->free_list.begin(), p->free_list.end(), out);
  return ok();
}

kv_status kv_pool_refcounts(const kv_pool* p, int32_t* out) {
  if (!p || !out) return fail(KV_ERR_INVALID, "NULL argument");
  std::copy(p->ref.begin(), p->ref.end(), out);
  return ok();
}

// ---- host tier ([KVM] asynchronous paged swap) ------------------------------

uint64_t kv_host_frame_bytes(const kv_pool* p) { return p ? static_cast<uint64_t>(frame_bytes(p->cfg)) : 0; }

kv_status kv_pool_attach_host(kv_pool* p, void* host_frames, int32_t n_frames, const int32_t* initial_free_order) {
  if (!p) return fail(KV_ERR_INVALID, "pool is NULL");
  if (p->n_frames > 0) return fail(KV_ERR_INVALID, "a host tier is already attached");
  if (n_frames <= 0) return fail(KV_ERR_INVALID, "n_frames must be positive");
  std::vector<int32_t> order(n_frames);
  if (initial_free_order) {
    std::vector<char> seen(n_frames, 0);
    for (int32_t i = 0; i < n_frames; ++i) {
      const int32_t f = initial_free_order[i];
      if (f < 0 || f >= n_frames || seen[f])
        return fail(KV_ERR_INVALID, "initial_free_order is not a permutation of the frame ids");
      seen[f] = 1;
      order[i] = f;
    }
  } else {
    std::iota(order.begin(), order.end(), 0);
  }
  p->host_frames = host_frames;
  p->n_frames = n_frames;
  p->host_free.assign(order.begin(), order.end());
  return ok();
}

namespace {

struct swap_undo {
  int64_t seq;
  kv_seq_state before;
  std::vector<int32_t> taken;  // frames (out) or blocks (in) popped from the front, in order
};

// Host bookkeeping of a swap-out: frames from the front of the host free list
// for every entry the sequence holds alone, in table order; the blocks lose
// their reference.  Returns the (block, frame) pairs; the blocks are the
// pairs' first members.
kv_status swap_out_plan(kv_pool* p, int64_t seq, int32_t* pairs_out, int32_t cap, int32_t* n_out, swap_undo& u) {
  if (!p) return fail(KV_ERR_INVALID, "pool is NULL");
  if (!n_out) return fail(KV_ERR_INVALID, "n_out is NULL");
  if (p->n_frames == 0) return fail(KV_ERR_INVALID, "no host tier attached");
  auto it = p->seqs.find(seq);
  if (it == p->seqs.end()) return fail(KV_ERR_INVALID, "unknown sequence " + std::to_string(seq));
  kv_seq_state& s = it->second;
  if (kv_status r = resident(s, seq)) return r;
  int32_t moved = 0;
  for (int32_t b : s.table) moved += p->ref[b] == 1;
  if (moved > cap || (moved > 0 && !pairs_out)) return fail(KV_ERR_INVALID, "pairs_out capacity too small");
  reclaim_ready(p, false);
  if (moved > static_cast<int32_t>(p->host_free.size()))
    return fail(KV_ERR_OOM, "no free host frame: " + std::to_string(moved) + " needed, " +
                                std::to_string(p->host_free.size()) + " free, " +
                                std::to_string(p->n_host_pending) + " pending");
  u.seq = seq;
  u.before = s;
  int32_t k = 0;
  if (moved > 0) s.host.assign(s.table.size(), -1);
  for (size_t j = 0; j < s.table.size(); ++j) {
    const int32_t b = s.table[j];
    if (p->ref[b] != 1) continue;
    const int32_t f = p->host_free.front();
    p->host_free.pop_front();
    u.taken.push_back(f);
    p->ref[b] = 0;
    s.host[j] = f;
    s.table[j] = -1;
    pairs_out[2 * k] = b;
    pairs_out[2 * k + 1] = f;
    ++k;
  }
  s.n_host = moved;
  *n_out = moved;
  return KV_OK;
}

void swap_out_undo(kv_pool* p, const swap_undo& u) {
  kv_seq_state& s = p->seqs[u.seq];
  for (int32_t b : u.before.table) p->ref[b] += (p->ref[b] == 0);
  for (auto f = u.taken.rbegin(); f != u.taken.rend(); ++f) p->host_free.push_front(*f);
  s = u.before;
}

// Host bookkeeping of a swap-in: a block from the front of the free list for
// every host-resident entry, in table order, all or nothing.  Returns the
// (frame, block) pairs.
kv_status swap_in_plan(kv_pool* p, int64_t seq, int32_t* pairs_out, int32_t cap, int32_t* n_out, swap_undo& u) {
  if (!p) return fail(KV_ERR_INVALID, "pool is NULL");
  if (!n_out) return fail(KV_ERR_INVALID, "n_out is NULL");
  auto it = p->seqs.find(seq);
  if (it == p->seqs.end()) return fail(KV_ERR_INVALID, "unknown sequence " + std::to_string(seq));
  kv_seq_state& s = it->second;
  if (s.n_host > cap || (s.n_host > 0 && !pairs_out)) return fail(KV_ERR_INVALID, "pairs_out capacity too small");
  reclaim_ready(p, false);
  if (s.n_host > static_cast<int32_t>(p->free_list.size()))
    return fail(KV_ERR_OOM, "no free KV block: " + std::to_string(s.n_host) + " needed, " +
                                std::to_string(p->free_list.size()) + " free, " + std::to_string(p->n_pending) +
                                " pending release");
  u.seq = seq;
  u.before = s;
  int32_t k = 0;
  for (size_t j = 0; j < s.table.size() && s.n_host > 0; ++j) {
    if (s.host[j] < 0) continue;
    const int32_t b = p->free_list.front();
    p->free_list.pop_front();
    u.taken.push_back(b);
    p->ref[b] = 1;
    s.table[j] = b;
    pairs_out[2 * k] = s.host[j];
    pairs_out[2 * k + 1] = b;
    ++k;
  }
  s.host.clear();
  s.n_host = 0;
  *n_out = k;
  return KV_OK;
}

void swap_in_undo(kv_pool* p, const swap_undo& u) {
  for (auto b = u.taken.rbegin(); b != u.taken.rend(); ++b) {
    p->ref[*b] = 0;
    p->free_list.push_front(*b);
  }
  p->seqs[u.seq] = u.before;
}

// The pending group of a swap: the blocks (out) or frames (in) named by the
// pairs' first members go back once the fence or event says the copy is done.
void swap_release(kv_pool* p, const int32_t* pairs, int32_t n, bool out, void* event, uint64_t fence,
                  bool immediate) {
  kv_pending_group g;
  g.event = event;
  g.fence = fence;
  for (int32_t i = 0; i < n; ++i) (out ? g.blocks : g.frames).push_back(pairs[2 * i]);
  if (immediate) {
    for (int32_t b : g.blocks) p->free_list.push_back(b);
    for (int32_t f : g.frames) p->host_free.push_back(f);
    return;
  }
  p->n_pending += static_cast<int32_t>(g.blocks.size());
  p->n_host_pending += static_cast<int32_t>(g.frames.size());
  p->pending.push_back(std::move(g));
}

kv_status swap_device(kv_pool* p, int64_t seq, bool out, void* d_staging, uint64_t staging_bytes, void* hip_stream,
                      int32_t* pairs_out, int32_t cap, int32_t* n_out) {
  if (!p) return fail(KV_ERR_INVALID, "pool is NULL");
  if (!p->host_frames || !p->k_cache || !p->v_cache)
    return fail(KV_ERR_INVALID, "the pool or its host tier has no memory to copy");
  if (!d_staging || staging_bytes < static_cast<uint64_t>(frame_bytes(p->cfg)))
    return fail(KV_ERR_INVALID, "staging buffer missing or smaller than one frame (" +
                                    std::to_string(frame_bytes(p->cfg)) + " bytes)");
  swap_undo u;
  if (kv_status r = out ? swap_out_plan(p, seq, pairs_out, cap, n_out, u) : swap_in_plan(p, seq, pairs_out, cap, n_out, u))
    return r;
  const int32_t n = *n_out;
  if (n == 0) return ok();
  if (kv_status r = swap_copy(p, pairs_out, n, out ? 0 : 1, d_staging, staging_bytes,
                              static_cast<hipStream_t>(hip_stream))) {
    out ? swap_out_undo(p, u) : swap_in_undo(p, u);
    *n_out = 0;
    return r;
  }
  void* ev = nullptr;
  if (kv_status r = record_event(hip_stream, &ev)) {
    // the copies are enqueued: the blocks or frames they read stay out of reach for good
    (void)hipStreamSynchronize(static_cast<hipStream_t>(hip_stream));
    swap_release(p, pairs_out, n, out, nullptr, 0, true);
    return r;
  }
  swap_release(p, pairs_out, n, out, ev, 0, false);
  return ok();
}

}  // namespace

kv_status kv_seq_swap_out_fenced(kv_pool* p, int64_t seq, uint64_t fence, int32_t* pairs_out, int32_t cap,
                                 int32_t* n_out) {
  swap_undo u;
  if (kv_status r = swap_out_plan(p, seq, pairs_out, cap, n_out, u)) return r;
  swap_release(p, pairs_out, *n_out, true, nullptr, fence, fence == 0);
  return ok();
}

kv_status kv_seq_swap_in_fenced(kv_pool* p, int64_t seq, uint64_t fence, int32_t* pairs_out, int32_t cap,
                                int32_t* n_out) {
  swap_undo u;
  if (kv_status r = swap_in_plan(p, seq, pairs_out, cap, n_out, u)) return r;
  swap_release(p, pairs_out, *n_out, false, nullptr, fence, fence == 0);
  return ok();
}

kv_status kv_seq_swap_out(kv_pool* p, int64_t seq, void* d_staging, uint64_t staging_bytes, void* hip_stream,
                          int32_t* pairs_out, int32_t cap, int32_t* n_out) {
  return swap_device(p, seq, true, d_staging, staging_bytes, hip_stream, pairs_out, cap, n_out);
}

kv_status kv_seq_swap_in(kv_pool* p, int64_t seq, void* d_staging, uint64_t staging_bytes, void* hip_stream,
                         int32_t* pairs_out, int32_t cap, int32_t* n_out) {
  return swap_device(p, seq, false, d_staging, staging_bytes, hip_stream, pairs_out, cap, n_out);
}

kv_status kv_swap_copy(kv_pool* p, const int32_t* pairs, int32_t n, int32_t direction, void* d_staging,
                       uint64_t staging_bytes, void* hip_stream) {
  if (!p) return fail(KV_ERR_INVALID, "pool is NULL");
  if (n < 0 || (n > 0 && !pairs)) return fail(KV_ERR_INVALID, "bad pair list");
  if (direction != 0 && direction != 1) return fail(KV_ERR_INVALID, "direction must be 0 (out) or 1 (in)");
  if (n == 0) return ok();
  if (!p->host_frames || !p->k_cache || !p->v_cache)
    return fail(KV_ERR_INVALID, "the pool or its host tier has no memory to copy");
  if (!d_staging || staging_bytes < static_cast<uint64_t>(frame_bytes(p->cfg)))
    return fail(KV_ERR_INVALID, "staging buffer missing or smaller than one frame (" +
                                    std::to_string(frame_bytes(p->cfg)) + " bytes)");
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = pairs[2 * i + direction], f = pairs[2 * i + 1 - direction];
    if (b < 0 || b >= p->cfg.num_blocks || f < 0 || f >= p->n_frames)
      return fail(KV_ERR_INVALID, "pair " + std::to_string(i) + " names a block or frame out of range");
  }
  return swap_copy(p, pairs, n, direction, d_staging, staging_bytes, static_cast<hipStream_t>(hip_stream));
}

kv_status kv_seq_residency(const kv_pool* p, int64_t seq, int32_t cap, int32_t* tier_out, int32_t* index_out,
                           int32_t* n_out) {
  if (!p || !n_out) return fail(KV_ERR_INVALID, "NULL argument");
  auto it = p->seqs.find(seq);
  if (it == p->seqs.end()) return fail(KV_ERR_INVALID, "unknown sequence " + std::to_string(seq));
  const kv_seq_state& s = it->second;
  const int32_t n = static_cast<int32_t>(s.table.size());
  *n_out = n;
  if (cap < n || (n > 0 && (!tier_out || !index_out))) return fail(KV_ERR_INVALID, "capacity too small");
  for (int32_t j = 0; j < n; ++j) {
    const bool host = s.n_host > 0 && s.host[j] >= 0;
    tier_out[j] = host ? KV_TIER_HOST : KV_TIER_HBM;
    index_out[j] = host ? s.host[j] : s.table[j];
  }
  return ok();
}

kv_status kv_host_free_list(const kv_pool* p, int32_t cap, int32_t* out, int32_t* n_out) {
  if (!p || !n_out) return fail(KV_ERR_INVALID, "NULL argument");
  const int32_t n = static_cast<int32_t>(p->host_free.size());
  *n_out = n;
  if (cap < n || (n > 0 && !out)) return fail(KV_ERR_INVALID, "capacity too small");
  std::copy(p->host_free.begin(), p->host_free.end(), out);
  return ok();
}

kv_status kv_pool_check(const kv_pool* p) {
  if (!p) return fail(KV_ERR_INVALID, "pool is NULL");
  const int32_t n = p->cfg.num_blocks;
  const int32_t B = p->cfg.block_size;
  std::vector<int32_t> counted(n, 0);
  for (const auto& kv : p->seqs) {
    const kv_seq_state& s = kv.second;
    if (static_cast<int64_t>(s.table.size()) != ceil_div(s.length, B))
      return fail(KV_ERR_STATE, "sequence " + std::to_string(kv.first) + " has a table of the wrong length");
    if (s.n_host > 0 && s.host.size() != s.table.size())
      return fail(KV_ERR_STATE, "sequence " + std::to_string(kv.first) + " has a residency list of the wrong length");
    int32_t n_host = 0;
    for (size_t j = 0; j < s.table.size(); ++j) {
      if (!s.host.empty() && s.host[j] >= 0) {
        if (s.table[j] != -1) return fail(KV_ERR_STATE, "an entry is resident in both tiers");
        ++n_host;
        continue;
      }
      const int32_t b = s.table[j];
      if (b < 0 || b >= n) return fail(KV_ERR_STATE, "table entry out of range");
      counted[b] += 1;
    }
    if (n_host != s.n_host) return fail(KV_ERR_STATE, "host entry count mismatch");
  }
  // host frames: free + pending + used by host entries = all frames, each once
  {
    std::vector<char> used(p->n_frames, 0);
    auto mark = [&](int32_t f) {
      if (f < 0 || f >= p->n_frames || used[f]) return false;
      used[f] = 1;
      return true;
    };
    int32_t count = 0, pend_f = 0;
    for (int32_t f : p->host_free) {
      if (!mark(f)) return fail(KV_ERR_STATE, "host free list holds a duplicate or invalid frame");
      ++count;
    }
    for (const auto& g : p->pending)
      for (int32_t f : g.frames) {
        if (!mark(f)) return fail(KV_ERR_STATE, "pending frame also free, used or pending twice");
        ++count;
        ++pend_f;
      }
    for (const auto& kv : p->seqs)
      if (kv.second.n_host > 0)
        for (int32_t f : kv.second.host)
          if (f >= 0) {
            if (!mark(f)) return fail(KV_ERR_STATE, "host frame used twice or invalid");
            ++count;
          }
    if (pend_f != p->n_host_pending) return fail(KV_ERR_STATE, "pending frame count mismatch");
    if (count != p->n_frames) return fail(KV_ERR_STATE, "free + pending + used frames != all frames");
  }
  for (int32_t b = 0; b < n; ++b)
    if (counted[b] + prefix_held(p, b) != p->ref[b])
      return fail(KV_ERR_STATE, "reference count of block " + std::to_string(b) +
                                    " disagrees with the tables and the prefix cache");
  std::vector<char> state(n, 0);  // 1 free, 2 pending
  for (int32_t b : p->free_list) {
    if (b < 0 || b >= n || state[b]) return fail(KV_ERR_STATE, "free list holds a duplicate or invalid block");
    state[b] = 1;
  }
  int32_t pend = 0;
  for (const auto& g : p->pending)
    for (int32_t b : g.blocks) {
      if (state[b]) return fail(KV_ERR_STATE, "pending block also free or pending twice");
      state[b] = 2;
      ++pend;
    }
  if (pend != p->n_pending) return fail(KV_ERR_STATE, "pending count mismatch");
  int32_t allocated = 0;
  for (int32_t b = 0; b < n; ++b) {
    if (p->ref[b] > 0) {
      ++allocated;
      if (state[b]) return fail(KV_ERR_STATE, "block " + std::to_string(b) + " is referenced but free or pending");
    }
  }
  if (static_cast<int32_t>(p->free_list.size()) + allocated + pend != n)
    return fail(KV_ERR_STATE, "N_free + N_allocated + N_pending != N_total");
  return ok();
}

}  // extern "C"
