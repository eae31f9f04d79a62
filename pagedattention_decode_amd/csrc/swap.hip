// Device side of the host tier: whole blocks between the pool and pinned host
// frames.
//
// [KVM] asynchronous paged swap (Figure 11 and the migration steps): the
// bytes cross the host link by DMA on a dedicated copy stream, so the copy
// engines move them while the compute units keep decoding.  A block is not
// contiguous in the pool (each layer's tiles of it are one run of Hkv tiles,
// a layer apart), and one DMA per run would cost a call per 2 L runs per
// block.  So the frames of a chunk are first packed into a contiguous device
// staging buffer by a copy kernel (HBM to HBM, far faster than the link), and
// the staging buffer goes to the frames with one DMA per run of consecutive
// frames; swap-in is the reverse.  Everything is enqueued on one stream, so
// a chunk's kernel waits for the previous chunk's DMA to release the staging
// buffer.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <string>

#include "pool_internal.h"

namespace pagedkv {
namespace {

constexpr int kSwapChunk = 256;  // frames per launch: their blocks travel in the kernel arguments
constexpr int kSwapThreads = 256;

struct swap_args {
  uint4* k;            // pool buffers (vectors of 16 bytes)
  uint4* v;
  uint4* staging;      // frame j of the chunk at j * 2 L * chunk_vec
  int64_t chunk_vec;   // one layer's Hkv tiles of one block, in vectors
  int64_t layer_vec;   // one layer of the pool: N * chunk_vec
  int32_t layers;      // L
  int32_t n;           // frames in this chunk
  int32_t blocks[kSwapChunk];
};

// One workgroup per run (frame j, layer l, K or V) at a time: the run's
// chunk_vec vectors are copied by consecutive threads, so both sides are read
// and written in whole 16-byte vectors, coalesced.  OUT: pool -> staging.
template <bool OUT>
__global__ void __launch_bounds__(kSwapThreads) swap_kernel(swap_args a) {
  const int64_t runs = static_cast<int64_t>(a.n) * 2 * a.layers;
  for (int64_t run = blockIdx.x; run < runs; run += gridDim.x) {
    const int j = static_cast<int>(run / (2 * a.layers));
    const int lk = static_cast<int>(run - static_cast<int64_t>(j) * 2 * a.layers);  // 2 l + (V ? 1 : 0)
    uint4* pool = (lk & 1) ? a.v : a.k;
    uint4* p = pool + static_cast<int64_t>(lk >> 1) * a.layer_vec + static_cast<int64_t>(a.blocks[j]) * a.chunk_vec;
    uint4* s = a.staging + run * a.chunk_vec;
    for (int64_t e = threadIdx.x; e < a.chunk_vec; e += kSwapThreads) {
      if constexpr (OUT)
        s[e] = p[e];
      else
        p[e] = s[e];
    }
  }
}

}  // namespace

kv_status swap_copy(kv_pool* pool, const int32_t* pairs, int32_t n, int32_t direction, void* d_staging,
                    uint64_t staging_bytes, hipStream_t st) {
  const kv_pool_config& c = pool->cfg;
  const int64_t F = frame_bytes(c);
  if (reinterpret_cast<uintptr_t>(d_staging) & 15) return fail(KV_ERR_INVALID, "staging must be 16-byte aligned");
  const int per = static_cast<int>(std::min<uint64_t>(staging_bytes / static_cast<uint64_t>(F), kSwapChunk));
  const bool out = direction == 0;
  char* host = static_cast<char*>(pool->host_frames);
  char* staging = static_cast<char*>(d_staging);
  swap_args a{};
  a.k = static_cast<uint4*>(pool->k_cache);
  a.v = static_cast<uint4*>(pool->v_cache);
  a.staging = static_cast<uint4*>(d_staging);
  a.chunk_vec = static_cast<int64_t>(c.num_kv_heads) * tile_bytes(c) / 16;
  a.layer_vec = static_cast<int64_t>(c.num_blocks) * a.chunk_vec;
  a.layers = c.num_layers;
  auto frame_of = [&](int i) { return pairs[2 * i + (out ? 1 : 0)]; };
  auto block_of = [&](int i) { return pairs[2 * i + (out ? 0 : 1)]; };
  // one DMA per run of consecutive frames of the chunk [i0, i0 + m)
  auto dma = [&](int i0, int m) -> kv_status {
    for (int j0 = 0; j0 < m;) {
      int j1 = j0 + 1;
      while (j1 < m && frame_of(i0 + j1) == frame_of(i0 + j1 - 1) + 1) ++j1;
      char* h = host + static_cast<int64_t>(frame_of(i0 + j0)) * F;
      char* d = staging + static_cast<int64_t>(j0) * F;
      const size_t bytes = static_cast<size_t>(j1 - j0) * F;
      hipError_t e = out ? hipMemcpyAsync(h, d, bytes, hipMemcpyDeviceToHost, st)
                         : hipMemcpyAsync(d, h, bytes, hipMemcpyHostToDevice, st);
      if (kv_status s = hip_check(e, "swap DMA")) return s;
      j0 = j1;
    }
    return KV_OK;
  };
  for (int i0 = 0; i0 < n; i0 += per) {
    const int m = std::min(per, n - i0);
    a.n = m;
    for (int j = 0; j < m; ++j) a.blocks[j] = block_of(i0 + j);
    if (!out)
      if (kv_status s = dma(i0, m)) return s;
    const int64_t runs = static_cast<int64_t>(m) * 2 * c.num_layers;
    const unsigned grid = static_cast<unsigned>(std::min<int64_t>(runs, 8192));
    if (out)
      hipLaunchKernelGGL(swap_kernel<true>, dim3(grid), dim3(kSwapThreads), 0, st, a);
    else
      hipLaunchKernelGGL(swap_kernel<false>, dim3(grid), dim3(kSwapThreads), 0, st, a);
    if (kv_status s = hip_check(hipGetLastError(), "swap kernel launch")) return s;
    if (out)
      if (kv_status s = dma(i0, m)) return s;
  }
  return KV_OK;
}

}  // namespace pagedkv
