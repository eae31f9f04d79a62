// Radix-tree prefix cache over the host block manager.
//
// Source (by page title): [KVM] "KV 缓存管理", cross-turn prefix caching —
// Table 2 (node: token run, ordered block ids, children, parent, ref_count,
// last_access), Definition 0.2, longest prefix match with block-aligned
// truncation (S_usable = floor(S_match / B) * B, the tail recomputed), and
// leaf-first LRU eviction of dormant nodes with cascading candidacy (Figure 6
// and the four eviction steps).
//
// Only full blocks are shared, so every edge holds whole blocks and a child is
// keyed by the tokens of its first block.  The tree holds one reference on
// every block it caches (counted in kv_pool::ref and, separately, in
// kv_prefix_tree::held); a request that attaches to a cached path, or inserts
// its own prefix, holds one ref_count on each node of that path until it is
// released.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <map>
#include <string>
#include <unordered_map>
#include <vector>

#include "pool_internal.h"

struct kv_prefix_node {
  std::vector<int32_t> tokens;  // a whole number of blocks
  std::vector<int32_t> blocks;  // tokens.size() / B physical blocks
  std::map<std::vector<int32_t>, kv_prefix_node*> children;  // keyed by the first block's tokens
  kv_prefix_node* parent = nullptr;
  int32_t ref_count = 0;
  uint64_t last_access = 0;
  uint64_t order = 0;  // creation order, the tie-break between equal access times
};

struct kv_prefix_tree {
  kv_prefix_node root;
  uint64_t clock = 0;
  uint64_t created = 0;
  std::unordered_map<int64_t, std::vector<kv_prefix_node*>> pins;  // request -> nodes it holds
  std::vector<int32_t> held;                                       // per block: references of the tree
};

namespace pagedkv {
namespace {

void free_subtree(kv_prefix_node* n) {
  for (auto& kv : n->children) {
    free_subtree(kv.second);
    delete kv.second;
  }
  n->children.clear();
}

kv_prefix_tree* tree_of(kv_pool* p) {
  if (!p->tree) {
    p->tree = new kv_prefix_tree();
    p->tree->held.assign(p->cfg.num_blocks, 0);
  }
  return p->tree;
}

std::vector<int32_t> key_at(const int32_t* tokens, int64_t at, int32_t B) {
  return std::vector<int32_t>(tokens + at, tokens + at + B);
}

bool block_equal(const std::vector<int32_t>& edge, int64_t e, const int32_t* tokens, int64_t at, int32_t B) {
  return std::equal(edge.begin() + e * B, edge.begin() + (e + 1) * B, tokens + at);
}

// Walk along whole edges matching tokens[0, n) block by block.  Returns the
// nodes fully matched, the blocks gathered, and where it stopped: (node,
// edge blocks matched) with matched = -1 when it stopped at a node boundary.
struct walk_result {
  std::vector<kv_prefix_node*> path;
  std::vector<int32_t> blocks;
  kv_prefix_node* stop = nullptr;
  int64_t matched = -1;
};

walk_result walk(kv_prefix_tree* t, const int32_t* tokens, int64_t n, int32_t B) {
  walk_result w;
  kv_prefix_node* node = &t->root;
  int64_t at = 0;
  while (at + B <= n) {
    auto it = node->children.find(key_at(tokens, at, B));
    if (it == node->children.end()) break;
    kv_prefix_node* child = it->second;
    int64_t e = 0;
    const int64_t edge_blocks = static_cast<int64_t>(child->blocks.size());
    while (e < edge_blocks && at + B <= n && block_equal(child->tokens, e, tokens, at, B)) {
      ++e;
      at += B;
    }
    w.blocks.insert(w.blocks.end(), child->blocks.begin(), child->blocks.begin() + e);
    if (e < edge_blocks) {
      w.stop = child;
      w.matched = e;
      return w;
    }
    w.path.push_back(child);
    node = child;
  }
  w.stop = node;
  w.matched = -1;
  return w;
}

void pin(kv_prefix_tree* t, int64_t seq, kv_prefix_node* n) {
  auto& v = t->pins[seq];
  if (std::find(v.begin(), v.end(), n) != v.end()) return;
  v.push_back(n);
  n->ref_count += 1;
}

}  // namespace

// Called when a request is released: it gives back its nodes' ref_counts.
void prefix_on_release(kv_pool* p, int64_t seq) {
  if (!p->tree) return;
  auto it = p->tree->pins.find(seq);
  if (it == p->tree->pins.end()) return;
  for (kv_prefix_node* n : it->second) n->ref_count -= 1;
  p->tree->pins.erase(it);
}

void prefix_destroy(kv_pool* p) {
  if (!p->tree) return;
  free_subtree(&p->tree->root);
  delete p->tree;
  p->tree = nullptr;
}

int32_t prefix_held(const kv_pool* p, int32_t block) { return p->tree ? p->tree->held[block] : 0; }

}  // namespace pagedkv

using namespace pagedkv;

extern "C" {

kv_status kv_prefix_match(kv_pool* p, const int32_t* tokens, int32_t n, int32_t* s_match, int32_t* s_usable) {
  if (!p || !s_match || !s_usable || (n > 0 && !tokens)) return fail(KV_ERR_INVALID, "NULL argument");
  if (n < 0) return fail(KV_ERR_INVALID, "n < 0");
  kv_prefix_tree* t = tree_of(p);
  const int32_t B = p->cfg.block_size;
  walk_result w = walk(t, tokens, n, B);
  const int64_t full = static_cast<int64_t>(w.blocks.size()) * B;
  // tokens matched inside the next block, which is not shared
  int64_t extra = 0;
  auto common = [&](const std::vector<int32_t>& edge, int64_t from) {
    int64_t k = 0;
    while (k < B && full + k < n && edge[from + k] == tokens[full + k]) ++k;
    extra = std::max(extra, k);
  };
  if (w.matched >= 0) {
    common(w.stop->tokens, w.matched * B);
  } else {
    for (auto& kv : w.stop->children) common(kv.second->tokens, 0);
  }
  const uint64_t now = ++t->clock;
  for (kv_prefix_node* nd : w.path) nd->last_access = now;
  if (w.matched >= 0) w.stop->last_access = now;
  *s_match = static_cast<int32_t>(full + extra);
  *s_usable = static_cast<int32_t>(full);
  return KV_OK;
}

kv_status kv_seq_attach_prefix(kv_pool* p, int64_t seq_id, const int32_t* tokens, int32_t n, int32_t* cached) {
  if (!p || !cached || (n > 0 && !tokens)) return fail(KV_ERR_INVALID, "NULL argument");
  if (n < 0) return fail(KV_ERR_INVALID, "n < 0");
  if (p->seqs.count(seq_id)) return fail(KV_ERR_INVALID, "sequence " + std::to_string(seq_id) + " exists");
  kv_prefix_tree* t = tree_of(p);
  const int32_t B = p->cfg.block_size;
  walk_result w = walk(t, tokens, n, B);
  kv_seq_state s;
  s.table = w.blocks;
  s.length = static_cast<int32_t>(w.blocks.size()) * B;
  for (int32_t b : s.table) p->ref[b] += 1;
  p->seqs.emplace(seq_id, std::move(s));
  const uint64_t now = ++t->clock;
  if (w.matched >= 0) w.path.push_back(w.stop);
  for (kv_prefix_node* nd : w.path) {
    pin(t, seq_id, nd);
    nd->last_access = now;
  }
  *cached = static_cast<int32_t>(w.blocks.size()) * B;
  return KV_OK;
}

kv_status kv_prefix_insert(kv_pool* p, int64_t seq_id, const int32_t* tokens, int32_t n, int32_t* cached) {
  if (!p || !cached || (n > 0 && !tokens)) return fail(KV_ERR_INVALID, "NULL argument");
  auto sit = p->seqs.find(seq_id);
  if (sit == p->seqs.end()) return fail(KV_ERR_INVALID, "unknown sequence " + std::to_string(seq_id));
  if (n < 0 || n > sit->second.length) return fail(KV_ERR_INVALID, "n must be in [0, sequence length]");
  if (sit->second.n_host > 0) return fail(KV_ERR_INVALID, "sequence " + std::to_string(seq_id) + " is swapped out");
  kv_prefix_tree* t = tree_of(p);
  const int32_t B = p->cfg.block_size;
  const std::vector<int32_t>& table = sit->second.table;
  const int64_t end = static_cast<int64_t>(n / B) * B;
  kv_prefix_node* node = &t->root;
  int64_t at = 0;
  std::vector<kv_prefix_node*> path;
  while (at < end) {
    auto it = node->children.find(key_at(tokens, at, B));
    if (it == node->children.end()) {
      auto* leaf = new kv_prefix_node();
      leaf->tokens.assign(tokens + at, tokens + end);
      leaf->blocks.assign(table.begin() + at / B, table.begin() + end / B);
      leaf->parent = node;
      leaf->order = ++t->created;
      for (int32_t b : leaf->blocks) {
        p->ref[b] += 1;
        t->held[b] += 1;
      }
      node->children.emplace(key_at(tokens, at, B), leaf);
      path.push_back(leaf);
      break;
    }
    kv_prefix_node* child = it->second;
    int64_t e = 0;
    const int64_t edge_blocks = static_cast<int64_t>(child->blocks.size());
    while (e < edge_blocks && at + B <= end && block_equal(child->tokens, e, tokens, at, B)) {
      ++e;
      at += B;
    }
    if (e < edge_blocks && at < end) {
      // the run diverges inside this edge: split it at the block boundary
      auto* upper = new kv_prefix_node();
      upper->tokens.assign(child->tokens.begin(), child->tokens.begin() + e * B);
      upper->blocks.assign(child->blocks.begin(), child->blocks.begin() + e);
      upper->parent = node;
      upper->ref_count = child->ref_count;
      upper->last_access = child->last_access;
      upper->order = ++t->created;
      for (auto& kv : t->pins)
        if (std::find(kv.second.begin(), kv.second.end(), child) != kv.second.end()) kv.second.push_back(upper);
      it->second = upper;  // same key: the first block is unchanged
      child->tokens.erase(child->tokens.begin(), child->tokens.begin() + e * B);
      child->blocks.erase(child->blocks.begin(), child->blocks.begin() + e);
      child->parent = upper;
      upper->children.emplace(std::vector<int32_t>(child->tokens.begin(), child->tokens.begin() + B), child);
      path.push_back(upper);
      node = upper;
      continue;
    }
    path.push_back(child);
    node = child;
  }
  const uint64_t now = ++t->clock;
  for (kv_prefix_node* nd : path) {
    nd->last_access = now;
    pin(t, seq_id, nd);
  }
  *cached = static_cast<int32_t>(end);
  return KV_OK;
}

static kv_status evict_common(kv_pool* p, int32_t target_free, void* event, uint64_t fence, bool immediate,
                              int32_t* blocks_out, int32_t cap, int32_t* n_out) {
  kv_prefix_tree* t = tree_of(p);
  std::vector<kv_prefix_node*> queue;
  std::vector<kv_prefix_node*> stack{&t->root};
  while (!stack.empty()) {
    kv_prefix_node* n = stack.back();
    stack.pop_back();
    for (auto& kv : n->children) stack.push_back(kv.second);
    if (n != &t->root && n->children.empty() && n->ref_count == 0) queue.push_back(n);
  }
  kv_pending_group g;
  g.event = event;
  g.fence = fence;
  std::vector<int32_t> evicted;
  auto available = [&] { return static_cast<int64_t>(p->free_list.size()) + static_cast<int64_t>(g.blocks.size()); };
  while (available() < target_free && !queue.empty()) {
    auto oldest = std::min_element(queue.begin(), queue.end(), [](const kv_prefix_node* a, const kv_prefix_node* b) {
      return a->last_access != b->last_access ? a->last_access < b->last_access : a->order < b->order;
    });
    kv_prefix_node* leaf = *oldest;
    queue.erase(oldest);
    for (int32_t b : leaf->blocks) {
      t->held[b] -= 1;
      p->ref[b] -= 1;
      if (p->ref[b] == 0) {
        if (immediate) p->free_list.push_back(b);
        else g.blocks.push_back(b);
      }
      evicted.push_back(b);
    }
    kv_prefix_node* parent = leaf->parent;
    parent->children.erase(std::vector<int32_t>(leaf->tokens.begin(), leaf->tokens.begin() + p->cfg.block_size));
    delete leaf;
    if (parent != &t->root && parent->children.empty() && parent->ref_count == 0) queue.push_back(parent);
  }
  if (!immediate) {
    if (g.blocks.empty()) {
      if (g.event) (void)hipEventDestroy(static_cast<hipEvent_t>(g.event));
    } else {
      p->n_pending += static_cast<int32_t>(g.blocks.size());
      p->pending.push_back(std::move(g));
    }
  }
  if (n_out) *n_out = static_cast<int32_t>(evicted.size());
  if (blocks_out)
    std::copy(evicted.begin(), evicted.begin() + std::min<size_t>(evicted.size(), std::max(cap, 0)), blocks_out);
  return KV_OK;
}

kv_status kv_prefix_evict(kv_pool* p, int32_t target_free, void* hip_stream, int32_t* blocks_out, int32_t cap,
                          int32_t* n_out) {
  if (!p) return fail(KV_ERR_INVALID, "pool is NULL");
  hipEvent_t ev = nullptr;
  hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
  if (e != hipSuccess) return fail(KV_ERR_HIP, std::string("hipEventCreateWithFlags: ") + hipGetErrorString(e));
  e = hipEventRecord(ev, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) {
    (void)hipEventDestroy(ev);
    return fail(KV_ERR_HIP, std::string("hipEventRecord: ") + hipGetErrorString(e));
  }
  return evict_common(p, target_free, ev, 0, false, blocks_out, cap, n_out);
}

kv_status kv_prefix_evict_fenced(kv_pool* p, int32_t target_free, uint64_t fence, int32_t* blocks_out, int32_t cap,
                                 int32_t* n_out) {
  if (!p) return fail(KV_ERR_INVALID, "pool is NULL");
  return evict_common(p, target_free, nullptr, fence, fence == 0, blocks_out, cap, n_out);
}

kv_status kv_prefix_stats(const kv_pool* p, int32_t* n_nodes, int32_t* n_cached_blocks, int32_t* n_pinned) {
  if (!p || !n_nodes || !n_cached_blocks || !n_pinned) return fail(KV_ERR_INVALID, "NULL argument");
  *n_nodes = *n_cached_blocks = *n_pinned = 0;
  if (!p->tree) return KV_OK;
  std::vector<const kv_prefix_node*> stack;
  for (auto& kv : p->tree->root.children) stack.push_back(kv.second);
  while (!stack.empty()) {
    const kv_prefix_node* n = stack.back();
    stack.pop_back();
    *n_nodes += 1;
    *n_cached_blocks += static_cast<int32_t>(n->blocks.size());
    if (n->ref_count > 0) *n_pinned += 1;
    for (auto& kv : n->children) stack.push_back(kv.second);
  }
  return KV_OK;
}

}  // extern "C"
