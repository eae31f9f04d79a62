// Stand-ins for the device side in the host-only sanitizer build (built by
// tests/test_host_sanitized.py with g++ and ASan/UBSan, together with pool.cpp and
// prefix_cache.cpp; never part of libpagedkv.so).  That build exercises the
// host block manager, the prefix cache and the host-tier bookkeeping on the
// CPU; every device entry point here fails with KV_ERR_UNSUPPORTED, so no
// computation can happen in it.

#include <hip/hip_runtime_api.h>

#include "pool_internal.h"

namespace pagedkv {

kv_status swap_copy(kv_pool*, const int32_t*, int32_t, int32_t, void*, uint64_t, hipStream_t) {
  return fail(KV_ERR_UNSUPPORTED, "host-only sanitizer build: no device code");
}

}  // namespace pagedkv

namespace {
kv_status no_device() { return pagedkv::fail(KV_ERR_UNSUPPORTED, "host-only sanitizer build: no device code"); }
}  // namespace

extern "C" {

kv_status reshape_and_cache(kv_pool*, int32_t, const void*, const void*, const int64_t*, int32_t, void*) {
  return no_device();
}

kv_status copy_blocks(kv_pool*, const int64_t*, int32_t, void*) { return no_device(); }

uint64_t paged_attention_workspace_bytes(const kv_pool*, int32_t, int32_t, int32_t, const kv_attention_options*) {
  return 0;
}

kv_status paged_attention_decode(kv_pool*, int32_t, const void*, void*, const int32_t*, const int32_t*, int32_t,
                                 int32_t, int32_t, const kv_attention_options*, void*, uint64_t, void*) {
  return no_device();
}

uint64_t paged_attention_static_scratch_bytes(void) { return 0; }

kv_status paged_attention_decode_static(kv_pool*, int32_t, const void*, void*, const int32_t*, const int32_t*,
                                        int32_t, int32_t, int32_t, const kv_attention_options*, void*) {
  return no_device();
}

uint64_t paged_attention_cascade_workspace_bytes(kv_pool*, int32_t, int32_t, int32_t, int32_t, int32_t,
                                                 const kv_attention_options*) {
  return 0;
}

kv_status paged_attention_decode_cascade(kv_pool*, int32_t, const void*, void*, const int32_t*, const int32_t*,
                                         int32_t, int32_t, int32_t, const int32_t*, const int32_t*, int32_t, int32_t,
                                         const kv_attention_options*, void*, uint64_t, void*) {
  return no_device();
}

uint64_t paged_prefill_workspace_bytes(const kv_pool*, int32_t, int32_t, int32_t, int32_t, int32_t,
                                       const kv_attention_options*) {
  return 0;
}

kv_status paged_attention_prefill(kv_pool*, int32_t, const void*, void*, const int32_t*, const int32_t*,
                                  const int32_t*, int32_t, int32_t, int32_t, int32_t, int32_t,
                                  const kv_attention_options*, void*, uint64_t, void*) {
  return no_device();
}

}  // extern "C"
