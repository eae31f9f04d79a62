// Internal view of a kv_pool shared by the host block manager (pool.cpp) and
// the device entry points (kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <deque>
#include <string>
#include <unordered_map>
#include <vector>

#include "pagedkv.h"

struct kv_prefix_tree;  // prefix_cache.cpp

struct kv_seq_state {
  std::vector<int32_t> table;  // logical block j -> physical block (-1 while host-resident)
  int32_t length = 0;          // tokens
  std::vector<int32_t> host;   // empty, or per entry: host frame of a host-resident entry, else -1
  int32_t n_host = 0;          // host-resident entries; > 0 means swapped out
};

struct kv_pending_group {
  void* event = nullptr;  // hipEvent_t, or nullptr for a fence group
  uint64_t fence = 0;     // used when event == nullptr
  bool ready = false;
  std::vector<int32_t> blocks;  // device blocks going back to the free list
  std::vector<int32_t> frames;  // host frames going back to the host free list
};

struct kv_pool {
  kv_pool_config cfg;
  void* k_cache = nullptr;
  void* v_cache = nullptr;
  std::deque<int32_t> free_list;             // pop front, push back
  std::vector<int32_t> ref;                  // per physical block
  std::unordered_map<int64_t, kv_seq_state> seqs;
  std::deque<kv_pending_group> pending;      // released, waiting for the device
  int32_t n_pending = 0;
  kv_prefix_tree* tree = nullptr;            // prefix cache, created on first use
  // host tier (kv_pool_attach_host): caller-owned pinned frames, FIFO free list
  void* host_frames = nullptr;
  int32_t n_frames = 0;
  std::deque<int32_t> host_free;
  int32_t n_host_pending = 0;
};

namespace pagedkv {

// Element size of an unquantised pool dtype (also of q / out / new rows of a
// quantised pool, which are bf16).
inline int elem_bytes(int32_t dtype) { return dtype == KV_F32 ? 4 : 2; }

inline bool is_quantized(int32_t dtype) { return dtype == KV_Q8_0 || dtype == KV_Q4_0; }

// Elements (values) of one (layer, block, kv head) tile.
inline int64_t tile_elems(const kv_pool_config& c) {
  return static_cast<int64_t>(c.block_size) * c.head_dim;
}

// Bytes of one (layer, block, kv head) tile of K (or of V): values, or codes
// plus one 2-byte scale per 32 values for a quantised pool.
inline int64_t tile_bytes(const kv_pool_config& c) {
  if (!is_quantized(c.dtype)) return tile_elems(c) * elem_bytes(c.dtype);
  const int bits = c.dtype == KV_Q8_0 ? 8 : 4;
  return tile_elems(c) * bits / 8 + tile_elems(c) / 32 * 2;
}

// Bytes of one host frame: the block's K tiles of every head, then its V
// tiles, for every layer in turn.
inline int64_t frame_bytes(const kv_pool_config& c) {
  return 2LL * c.num_layers * c.num_kv_heads * tile_bytes(c);
}

// Bytes of the whole K (or V) buffer.
inline int64_t pool_bytes(const kv_pool_config& c) {
  return static_cast<int64_t>(c.num_layers) * c.num_blocks * c.num_kv_heads * tile_bytes(c);
}

// Sets the thread-local error message and returns the status.
kv_status fail(kv_status st, const std::string& msg);

// Prefix cache hooks (prefix_cache.cpp).
void prefix_on_release(kv_pool* p, int64_t seq);  // the request gives back its nodes' ref_counts
void prefix_destroy(kv_pool* p);
int32_t prefix_held(const kv_pool* p, int32_t block);  // references the tree holds on a block

// Multi-query attention for the pools the multi-query kernel does not read
// (kernels.hip): one decode query per chunk row, through the decode kernels.
// q and out rows are in the pool's element type (bf16 for quantised pools).
uint64_t prefill_rowwise_workspace(const kv_pool* pool, int total_q, int num_q_heads, int max_blocks,
                                   const kv_attention_options* opts);
kv_status prefill_rowwise(kv_pool* pool, int layer, const void* q, void* out, const int32_t* q_indptr,
                          const int32_t* tables, const int32_t* ctx, int n_seqs, int total_q, int max_q_len,
                          int max_blocks, int num_q_heads, const kv_attention_options* opts, void* ws,
                          uint64_t ws_bytes, hipStream_t st);

// Device side of a swap (swap.hip): pairs are (block, frame) for direction 0
// (out) and (frame, block) for direction 1 (in); checked by the caller.
kv_status swap_copy(kv_pool* pool, const int32_t* pairs, int32_t n, int32_t direction, void* d_staging,
                    uint64_t staging_bytes, hipStream_t st);

// Shared by the attention entry points (defined with the decode kernels).
constexpr int kMaxGroup = 16;  // query heads per KV head
kv_status hip_check(hipError_t e, const char* what);
bool mfma_supported(const kv_pool_config& c, int G);  // bf16, B = 16, d in {64, 128, 256}, G <= 16
int device_cus();                                    // compute units of the current device
size_t max_lds_per_block();                          // LDS bytes a workgroup may use on the current device
uint64_t up256(uint64_t b);                          // rounded up to 256 bytes

// Timing events of a call (kv_timing_events), all null when none were given.
struct call_events {
  hipEvent_t start = nullptr, kernel_stop = nullptr, stop = nullptr;
};
inline call_events events_of(const kv_attention_options* o) {
  call_events e;
  if (o && o->timing) {
    e.start = static_cast<hipEvent_t>(o->timing->start);
    e.kernel_stop = static_cast<hipEvent_t>(o->timing->kernel_stop);
    e.stop = static_cast<hipEvent_t>(o->timing->stop);
  }
  return e;
}


}  // namespace pagedkv
