/*
 * pagedkv.h -- C ABI of a paged KV cache with single-query decode attention
 * for AMD Instinct MI355X (gfx950).
 *
 * The library keeps the host-side block manager of a paged KV cache (free
 * list, per-block reference counts, per-sequence block tables) and launches
 * HIP kernels that scatter new K/V rows into their slots, copy blocks for
 * copy-on-write, and compute decode attention by gathering each sequence's
 * keys and values through its block table.
 *
 * Sources, cited by page title:
 *   [KVM] "KV 缓存管理" (KV cache management chapter of an ML-systems book):
 *         Eq. 1 (per-token footprint); "Paged KV allocation" and its
 *         "PagedAttention virtual memory model" (block table T: l -> p,
 *         l = floor(t/B), o = t mod B, allocation when o = 0, M_block);
 *         "Zero-copy branching via copy-on-write" (fork, refcounts, CoW,
 *         reclamation); "Chunked prefill mechanism" (running-max merge).
 *   [BT]  "KV Cache 还有空间为何新请求却进不来？PagedAttention 的块表与碎片控制"
 *         (block tables and fragmentation): §03 translation, §04 growth,
 *         §05 block manager, §06 tensor shapes, §07 decode equation, §08 CoW,
 *         §10 atomic reservation, §13 conservation.
 *   [INF] "第 8 章 推理优化" (inference optimisation): §8.3.2 release only
 *         when no reference remains and no submitted device work reads it;
 *         §8.2.3 query-key pairs of a chunk; §8.5.1 verification of draft
 *         positions in one pass.
 *
 * Conventions for every call:
 *   - Status codes; on failure kv_last_error() returns a message (thread
 *     local) and no state has changed unless the call says otherwise.
 *   - The library owns host metadata only.  Every device pointer (pools, q,
 *     out, tables, slot mappings, workspace) is caller-owned device memory.
 *   - Device operations are enqueued on the given HIP stream (a hipStream_t
 *     passed as void*; NULL is the default stream) and never synchronise.
 *   - A pool is not thread safe: use it from one host thread at a time.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KV_OK = 0,
  KV_ERR_OOM = 1,         /* the free list cannot cover the request ([BT] §05) */
  KV_ERR_INVALID = 2,     /* bad argument, unknown or duplicate sequence */
  KV_ERR_STATE = 3,       /* internal invariant violated (kv_pool_check) */
  KV_ERR_HIP = 4,         /* a HIP runtime call failed; the message names it */
  KV_ERR_UNSUPPORTED = 5  /* valid but not implemented shape / dtype / kernel */
} kv_status;

/* KV_Q8_0, KV_Q4_0: the pool stores K and V quantised in groups of 32 values
 * with one 2-byte scale per group ([INF] §8.4.2, Figure 8-23: 34 and 18
 * bytes per 32 values); new rows, q and out are bf16.  Quantised pools need
 * B = 16 and d in {64, 128, 256}. */
typedef enum { KV_F32 = 0, KV_BF16 = 1, KV_Q8_0 = 2, KV_Q4_0 = 3 } kv_dtype;

typedef struct {
  int32_t num_layers;   /* L */
  int32_t num_blocks;   /* N physical blocks in the pool */
  int32_t block_size;   /* B tokens per block */
  int32_t num_kv_heads; /* Hkv */
  int32_t head_dim;     /* d; a multiple of 32, at most 256 */
  int32_t dtype;        /* kv_dtype of K and V (and of q and out unless quantised) */
} kv_pool_config;

typedef struct kv_pool kv_pool; /* opaque */

typedef struct {
  int32_t n_free;      /* blocks on the free list */
  int32_t n_allocated; /* blocks with reference count > 0 */
  int32_t n_shared;    /* blocks with reference count > 1 */
  int32_t n_pending;   /* released blocks waiting for device work to finish */
  int32_t n_seqs;      /* live sequences */
  int64_t n_tokens;    /* sum of live sequence lengths */
  int64_t n_table_refs;/* sum of live block-table lengths */
} kv_pool_stats_t;

/* ------------------------------------------------------------------------
 * Pool memory layout (the pages leave the stride open, [BT] §06).
 *
 * K and V are two separate caller-owned buffers, each holding, for every
 * (layer l, physical block p, KV head g), one contiguous tile of B*d
 * elements:
 *     tile(l, p, g) = ((l * N + p) * Hkv + g) * B * d          (elements)
 * Inside a tile, the element of slot r (0 <= r < B) and dimension e
 * (0 <= e < d) sits at
 *     K: tile + ((e / X) * B + r) * X + e % X,     X = 16 / sizeof(element)
 *     V: tile + ((((e / 32) * (B / Q) + r / Q) * 16 + e % 16) * 2
 *                + (e % 32) / 16) * Q + r % Q,      Q = gcd(B, 4)
 * so that one 16-byte load brings X dimensions of one key, or 4 slots of
 * two value dimensions 16 apart; these are the operand orders of the
 * gfx950 bf16 matrix instructions used by the decode kernel.
 *
 * Quantised pools (B = 16).  A value x of a group of 32 (32 consecutive
 * dimensions 32 g .. 32 g + 31 of one slot of one KV head) is stored as a code
 * c with x ~ c * s: s = max|x| / M (M = 127 for q8_0, 7 for q4_0) in float32,
 * rounded to the nearest IEEE half (saturating at 65504), and
 * c = rint(x / s) (float32 quotient, ties to even, clamped to [-M, M]; 0 when
 * s = 0).  A tile is T = 16 d bits/8 code bytes followed by 16 x d/32 scales
 * (half, at T + (r * d/32 + g) * 2), tile(l, p, g) = ((l * N + p) * Hkv + g) *
 * (T + d) bytes.  Codes sit per matrix-core lane L = 16 q + r (q < 4, r < 16),
 * which owns the d * bits / 32 bytes at L * d * bits / 32:
 *     K, lane (q, r): slot r, dims 32 k + 8 q + j (k < d/32, j < 8) at
 *         q8_0 byte 8 k + j; q4_0 byte 4 k + j % 4, low nibble for j < 4;
 *     V, lane (q, r): dim 16 t + r of slots 4 q + i (t < d/16, i < 4) at
 *         q8_0 byte 4 t + i; q4_0 byte 4 (t/2) + i, low nibble for even t.
 * q8_0 codes are two's-complement bytes, q4_0 codes are stored as c + 8.
 * ---------------------------------------------------------------------- */

/* Bytes the caller must allocate for the K and the V buffer. */
kv_status kv_pool_required_bytes(const kv_pool_config* cfg, uint64_t* k_bytes, uint64_t* v_bytes);

/* Create the host block manager over caller-owned device buffers k_cache and
 * v_cache (each kv_pool_required_bytes large, 256-byte aligned).  The free
 * list starts as initial_free_order (a permutation of 0..N-1; NULL means
 * 0, 1, ..., N-1) and is first-in first-out ([BT] §05).  All reference counts
 * start at zero.  The buffers are not touched and never freed by the library. */
kv_status kv_pool_create(const kv_pool_config* cfg, void* k_cache, void* v_cache,
                         const int32_t* initial_free_order, kv_pool** out);

/* Destroy the host state (and any pending release events). */
void kv_pool_destroy(kv_pool* pool);

/* The configuration the pool was created with (for callers that check tensor
 * shapes and element types against it). */
kv_status kv_pool_get_config(const kv_pool* pool, kv_pool_config* out);

/* Register an empty sequence: length 0 and an empty block table; its first
 * append allocates its first block ([BT] §05: a new request starts with no
 * blocks and a block is taken when the first token's offset is 0; [KVM] paged
 * KV allocation, allocation at o = 0).  KV_ERR_INVALID if seq_id exists. */
kv_status kv_seq_add(kv_pool* pool, int64_t seq_id);

/* Fork: child gets a copy of parent's block table, each of those blocks gains
 * one reference, child's length = parent's; no device work ([KVM] copy-on-write
 * branching, the table copy / refcount increment / registration steps). */
kv_status kv_seq_fork(kv_pool* pool, int64_t parent, int64_t child);

/* Append n_new[i] tokens to seq_ids[i] for i < n, sequence-major in the given
 * order, as one all-or-nothing batch ([BT] §10).  For each token, with
 * j = len / B and r = len % B ([BT] §03-§04):
 *   - j == table length: pop the front of the free list, append it (ref = 1);
 *   - else if ref[T[j]] > 1 (shared): pop p_new, emit the pair (T[j], p_new)
 *     into cow_pairs_out, drop one reference of T[j], set T[j] = p_new
 *     ([KVM] copy-on-write; [BT] §08);
 *   - write slot T[j] * B + r into slot_mapping_out; len += 1.
 * Outputs (host memory): slot_mapping_out[sum n_new] (capacity slot_capacity),
 * cow_pairs_out[n_cow][2] as (src, dst) (capacity cow_capacity pairs; n pairs
 * always suffice), *n_cow_out.  The caller must enqueue copy_blocks(pairs)
 * before reshape_and_cache on the same stream.  KV_ERR_OOM when the free list
 * runs dry: the whole batch is undone and no state changes.  Released blocks
 * whose device work has completed are returned to the free list first. */
kv_status kv_append_slots(kv_pool* pool, int32_t n, const int64_t* seq_ids, const int32_t* n_new,
                          int64_t* slot_mapping_out, int64_t slot_capacity,
                          int64_t* cow_pairs_out, int32_t cow_capacity, int32_t* n_cow_out);

/* Host copy of the block tables and lengths of n sequences, the per-sequence
 * logical -> physical block maps the decode kernel reads ([BT] §06: the
 * block_tables [num_seqs, max_blocks] and context_lens inputs of the decode;
 * [KVM] PagedAttention virtual memory model: T maps logical block l to
 * physical block p): tables_out[n][max_blocks] (row i, entries past
 * ceil(len/B) set to -1) and context_lens_out[n].  KV_ERR_INVALID if a table
 * is longer than max_blocks or a sequence is unknown or swapped out. */
kv_status kv_get_block_tables(const kv_pool* pool, int32_t n, const int64_t* seq_ids,
                              int32_t max_blocks, int32_t* tables_out, int32_t* context_lens_out);

/* Length in tokens and block-table length of one sequence. */
kv_status kv_seq_info(const kv_pool* pool, int64_t seq_id, int32_t* length, int32_t* num_blocks);

/* Release a sequence: each block of its table loses a reference.  Blocks that
 * reach zero return to the back of the free list, in table order, only after
 * all work enqueued so far on hip_stream has completed ([KVM] reclamation;
 * [INF] §8.3.2): an event is recorded on the stream and polled at the next
 * append or kv_pool_reclaim. */
kv_status kv_seq_release(kv_pool* pool, int64_t seq_id, void* hip_stream);

/* As kv_seq_release, with a caller-managed fence instead of a HIP event: the
 * freed blocks wait until kv_pool_retire(pool, f) is called with f >= fence.
 * fence == 0 returns them at once. */
kv_status kv_seq_release_fenced(kv_pool* pool, int64_t seq_id, uint64_t fence);

/* Declare every fence <= completed_fence done, then reclaim. */
kv_status kv_pool_retire(kv_pool* pool, uint64_t completed_fence);

/* Return released blocks whose events completed (wait != 0: wait for all
 * pending events first).  Ready groups go back in release order. */
kv_status kv_pool_reclaim(kv_pool* pool, int32_t wait);

/* Occupancy of the pool: the counts the conservation law of [BT] §13 relates
 * (N_free + N_allocated + N_pending = N_total), so that the KV-cache
 * utilisation U_KV = N_allocated / N_total of [KVM] (serving telemetry, Eq. 8)
 * can be monitored; the blocks held more than once ([KVM] copy-on-write
 * branching: shared blocks have a reference count above one); and the live
 * sequences' tokens and table entries (tokens / (entries * B) is the slot
 * occupancy, whose complement is the tail waste of [BT] §04).  Host memory; no
 * device work. */
kv_status kv_pool_stats(const kv_pool* pool, kv_pool_stats_t* out);

/* Free list in pop order (out capacity cap; *n_out = its length). */
kv_status kv_pool_free_list(const kv_pool* pool, int32_t cap, int32_t* out, int32_t* n_out);

/* Reference counts of all N blocks (out[N]). */
kv_status kv_pool_refcounts(const kv_pool* pool, int32_t* out);

/* Conservation ([BT] §13): N_free + N_allocated + N_pending = N_total, the set
 * of blocks with ref > 0 is exactly the set named by tables and the prefix
 * cache, each count equals the number of HBM-resident table entries naming the
 * block plus the prefix cache's reference, and every table has ceil(len / B)
 * entries; with a host tier, free + pending + host-resident frames are every
 * frame exactly once.  KV_ERR_STATE names the first violation. */
kv_status kv_pool_check(const kv_pool* pool);

/* ------------------------------------------------------------------------
 * Host tier: swap of a sequence's blocks to pinned host memory and back
 * ([KVM] asynchronous paged swap, Figure 11: frames of a pre-allocated pinned
 * host pool, the copy on a dedicated stream, the block table remapped with a
 * residency tag per entry, the device frames reused once the copy is done).
 *
 * A host frame holds one block of every layer: for l = 0 .. L-1, the block's
 * K tiles of all Hkv heads (Hkv tile bytes, as laid out in the pool), then its
 * V tiles; kv_host_frame_bytes = 2 L Hkv tile bytes = B times the per-token
 * footprint ([KVM] Eq. 1) for an unquantised pool.  Frame f starts at
 * host_frames + f * kv_host_frame_bytes.
 *
 * Only entries whose block the sequence holds alone (reference count 1) move;
 * a block shared with a fork or held by the prefix cache stays in HBM, still
 * referenced.  A sequence with a host-resident entry is "swapped out": it can
 * be released or swapped in, and kv_seq_info / kv_seq_residency answer for it;
 * append, fork, kv_get_block_tables, kv_shared_prefix_plan and
 * kv_prefix_insert refuse it (KV_ERR_INVALID).
 * ---------------------------------------------------------------------- */

typedef enum { KV_TIER_HBM = 0, KV_TIER_HOST = 1 } kv_tier;

/* Bytes of one host frame (0 for a NULL pool). */
uint64_t kv_host_frame_bytes(const kv_pool* pool);

/* Give the pool n_frames host frames at host_frames (caller-owned page-locked
 * memory, n_frames * kv_host_frame_bytes bytes, from hipHostMalloc or an
 * equivalent pinned allocation: pageable memory would stall the copies; NULL
 * allows host bookkeeping only).  The host free list starts as
 * initial_free_order (a permutation of 0..n_frames-1; NULL = 0, 1, ...) and is
 * first-in first-out.  Once per pool. */
kv_status kv_pool_attach_host(kv_pool* pool, void* host_frames, int32_t n_frames, const int32_t* initial_free_order);

/* Swap out: for every entry of the sequence's table whose block it holds alone,
 * in table order, take a frame from the front of the host free list, emit the
 * pair (block, frame) into pairs_out[n][2] (capacity cap pairs; the table
 * length always suffices), tag the entry as host-resident with that frame and
 * drop the block's reference.  All or nothing: KV_ERR_OOM when the host free
 * list is too short (nothing changes).  Enqueues on hip_stream the copies of
 * the blocks to their frames (through d_staging, a device buffer of at least
 * one frame, 16-byte aligned, used in chunks of whole frames); the blocks
 * return to the back of the free list once that work has completed (an event
 * polled like kv_seq_release's).  The caller orders hip_stream after the work
 * that wrote the blocks.  *n_out = number of pairs (0: nothing moved). */
kv_status kv_seq_swap_out(kv_pool* pool, int64_t seq_id, void* d_staging, uint64_t staging_bytes, void* hip_stream,
                          int32_t* pairs_out, int32_t cap, int32_t* n_out);

/* Swap in: for every host-resident entry, in table order, take a block from the
 * front of the free list, emit (frame, block), set the entry to the block
 * (reference 1).  All or nothing: KV_ERR_OOM when the free list is too short.
 * Enqueues the copies frames -> blocks on hip_stream; the frames return to the
 * back of the host free list once that work has completed.  Work that reads
 * the sequence must be ordered after hip_stream. */
kv_status kv_seq_swap_in(kv_pool* pool, int64_t seq_id, void* d_staging, uint64_t staging_bytes, void* hip_stream,
                         int32_t* pairs_out, int32_t cap, int32_t* n_out);

/* The same bookkeeping without device work: the blocks (out) or frames (in)
 * wait for kv_pool_retire(pool, f >= fence) (fence 0: at once).  The caller
 * moves the bytes with kv_swap_copy and retires the fence after it. */
kv_status kv_seq_swap_out_fenced(kv_pool* pool, int64_t seq_id, uint64_t fence, int32_t* pairs_out, int32_t cap,
                                 int32_t* n_out);
kv_status kv_seq_swap_in_fenced(kv_pool* pool, int64_t seq_id, uint64_t fence, int32_t* pairs_out, int32_t cap,
                                int32_t* n_out);

/* Device side only: copy n pairs (host memory) on hip_stream; direction 0 =
 * out, pairs (block, frame); direction 1 = in, pairs (frame, block).  Each
 * chunk of whole frames is gathered by a kernel into d_staging and moved by
 * one DMA copy per run of consecutive frames (out), or the reverse (in).
 * KV_ERR_INVALID for a block or frame out of range. */
kv_status kv_swap_copy(kv_pool* pool, const int32_t* pairs, int32_t n, int32_t direction, void* d_staging,
                       uint64_t staging_bytes, void* hip_stream);

/* The extended block table of a sequence: per entry, its tier (kv_tier) and
 * its block (KV_TIER_HBM) or frame (KV_TIER_HOST); capacity cap entries,
 * *n_out = table length. */
kv_status kv_seq_residency(const kv_pool* pool, int64_t seq_id, int32_t cap, int32_t* tier_out, int32_t* index_out,
                           int32_t* n_out);

/* Host free list in pop order. */
kv_status kv_host_free_list(const kv_pool* pool, int32_t cap, int32_t* out, int32_t* n_out);

/* Message of the last failed call on this thread ("" if none). */
const char* kv_last_error(void);

/* ------------------------------------------------------------------------
 * Prefix cache ([KVM] cross-turn prefix caching: Table 2, Definition 0.2,
 * Figure 6).  A radix tree binds runs of prompt tokens to the physical blocks
 * holding their K/V, so a later request with the same prefix reuses them
 * instead of recomputing them.  Only completely filled blocks are shared: a
 * match of S_match tokens gives S_usable = floor(S_match / B) * B cached
 * tokens and the tail is recomputed (block-aligned truncation).  Every edge
 * holds whole blocks; a child is keyed by the tokens of its first block.  The
 * tree holds one reference on each block it caches; a request attached to or
 * inserted into the tree holds a ref_count on each node of its path until it
 * is released.  Nodes with ref_count 0 are dormant; eviction takes dormant
 * leaves oldest last_access first, and a parent left childless and dormant
 * becomes a candidate in turn.  last_access is a counter advanced by every
 * lookup, attach and insert (ties go to the node created first).  Tokens are
 * int32 host arrays; the tree lives on the host.
 * ---------------------------------------------------------------------- */

/* Longest cached prefix of tokens[0, n): S_match tokens (whole blocks along
 * the tree plus the longest common run with the next block), of which
 * S_usable (whole blocks) can be reused.  Marks the walked nodes accessed. */
kv_status kv_prefix_match(kv_pool* pool, const int32_t* tokens, int32_t n, int32_t* s_match, int32_t* s_usable);

/* Register a new sequence whose table starts with the cached blocks of the
 * longest block-aligned prefix of tokens[0, n) (each gains a reference);
 * *cached_tokens = its length (a multiple of B).  The caller then appends and
 * computes the rest.  KV_ERR_INVALID if seq_id exists. */
kv_status kv_seq_attach_prefix(kv_pool* pool, int64_t seq_id, const int32_t* tokens, int32_t n,
                               int32_t* cached_tokens);

/* Cache the first floor(n / B) blocks of sequence seq_id, whose first n
 * tokens are tokens[0, n) and already hold their K/V.  Nodes the tree lacks
 * adopt the sequence's blocks (the tree takes a reference); a run diverging
 * inside an edge splits it at the block boundary.  n <= the sequence length. */
kv_status kv_prefix_insert(kv_pool* pool, int64_t seq_id, const int32_t* tokens, int32_t n, int32_t* cached_tokens);

/* Evict dormant leaves until the free list (plus blocks this call makes
 * pending) holds target_free blocks or no dormant leaf is left.  Blocks
 * whose last reference was the tree's go to the free list once the work
 * enqueued on hip_stream so far has completed (as kv_seq_release), or, for
 * the fenced form, once completed_fence >= fence (0 = at once).  The evicted
 * nodes' blocks, in eviction order, go to blocks_out (at most cap entries;
 * blocks_out may be NULL) and their number to *n_out. */
kv_status kv_prefix_evict(kv_pool* pool, int32_t target_free, void* hip_stream, int32_t* blocks_out, int32_t cap,
                          int32_t* n_out);
kv_status kv_prefix_evict_fenced(kv_pool* pool, int32_t target_free, uint64_t fence, int32_t* blocks_out,
                                 int32_t cap, int32_t* n_out);

/* Groups for paged_attention_decode_cascade from the host tables: maximal runs
 * of consecutive sequences of seq_ids[0, n) that share at least one completely
 * filled leading block with the run's first member; shared_blocks[g] = the
 * number of leading blocks every member has in common with it and completely
 * filled (0 for a run of one).  group_start needs n + 1 entries, shared_blocks
 * n; *n_groups receives the number of groups. */
kv_status kv_shared_prefix_plan(const kv_pool* pool, int32_t n, const int64_t* seq_ids, int32_t* group_start,
                                int32_t* shared_blocks, int32_t* n_groups);

/* Nodes, blocks cached by the tree, and pinned nodes (ref_count > 0). */
kv_status kv_prefix_stats(const kv_pool* pool, int32_t* n_nodes, int32_t* n_cached_blocks, int32_t* n_pinned);

/* ------------------------------------------------------------------------
 * Device operations
 * ---------------------------------------------------------------------- */

/* Scatter new key/value rows into the pool of one layer ([KVM] paged KV
 * allocation: the token's K and V go to T[l] at offset o; [BT] §11: decode
 * appends one KV slot per sequence).  k_new, v_new: device [n_tokens][Hkv][d]
 * in the pool dtype (bf16 for a quantised pool); d_slot_mapping: device
 * int64[n_tokens], slot = p * B + r.  Slots < 0 or >= N * B are skipped.
 * Bitwise copy, or quantisation as described above for q8_0 / q4_0 pools. */
kv_status reshape_and_cache(kv_pool* pool, int32_t layer, const void* k_new, const void* v_new,
                            const int64_t* d_slot_mapping, int32_t n_tokens, void* hip_stream);

/* Copy-on-write block copies ([KVM] CoW: the shared block's B tokens are copied
 * to p_new): for each pair (src, dst) of device int64[n_pairs][2], in every
 * layer, K and V tiles of dst become bitwise copies of src.  Pairs naming a
 * block outside [0, N) are skipped; the dst blocks must be distinct and no dst
 * may be a src of the same call. */
kv_status copy_blocks(kv_pool* pool, const int64_t* d_pairs, int32_t n_pairs, void* hip_stream);

typedef enum {
  KV_KERNEL_AUTO = 0,    /* the matrix-core kernel where it applies, else generic */
  KV_KERNEL_GENERIC = 1, /* vector-ALU kernel: f32 or bf16, any B, d; G <= 16 */
  KV_KERNEL_MFMA = 2     /* bf16 with B in {4, 8, 16, 32, 64}, or q8_0 / q4_0
                            with B = 16; d in {64, 128, 256}, G <= 16.  A call
                            of more than 4095 sequences runs as consecutive
                            launches over slices of at most 4095 (the
                            workspace holds one slice).  It works in 16-token
                            tiles: B/16 tiles per table entry for B > 16, 16/B
                            entries per tile for B < 16 (entries past a
                            context are never read).  The only kernel for
                            quantised pools (the codes, exact in bf16, are the
                            matrix operands and the group scales are applied in
                            float32: the result is the attention over
                            code x scale) */,
  KV_KERNEL_MFMA_STAGED_TABLE = 3 /* the matrix-core kernel (bf16, B = 16 only)
                            with each wave's block-table entries copied into
                            an LDS slice when its run starts (straight from
                            global memory, one wait) and read from there per
                            tile, instead of one scalar load per tile.  The
                            pages describe warps that load the block pointers
                            into shared memory or registers ([KVM]
                            PagedAttention virtual memory model); this
                            variant measures that choice against the scalar
                            loads of KV_KERNEL_MFMA.  Same results, bit for
                            bit */,
  KV_KERNEL_VALU = 4     /* the same split-K kernel (runs, register ring,
                            merge) with vector-ALU arithmetic instead of matrix
                            instructions: v_dot2_f32_bf16 scores over each
                            lane's dims summed by lane swaps, DPP row maxima,
                            weights gathered across lanes and v_dot2 over token
                            pairs for the values.  bf16, B = 16, d = 128,
                            G = 4 or 8.  It measures whether the matrix
                            instructions pay on a GQA group of at most 8 query
                            rows, which the pages leave open */
} kv_kernel;

/* Optional timing of an attention call.  Each field is a hipEvent_t that
 * already exists (created by the caller, e.g. a torch.cuda.Event recorded
 * once), or NULL.  The library attaches the events to its own kernel launches
 * (hipExtLaunchKernel), so they carry the GPU timestamps of the kernels
 * themselves and add no marker between kernels:
 *   start        start of the call's first kernel;
 *   kernel_stop  end of the kernel that streams the K/V cache -- the split-K
 *                partition kernel of paged_attention_decode and the
 *                multi-query kernel of paged_attention_prefill (both the
 *                call's first kernel, so start .. kernel_stop is that kernel
 *                alone; when a decode of more than 4095 sequences runs
 *                as several launches, start .. kernel_stop spans them),
 *                the fused prefix-and-suffix kernel of the cascade
 *                (also its first kernel), the
 *                last decode kernel of the row-wise prefill path (after its
 *                row-length kernel and any earlier batches);
 *   stop         end of the call's last kernel.
 * Where the last kernel is also the one that streams the cache (one-kernel
 * calls), stop is recorded right after it as an ordinary event.  The caller
 * owns the events; the library only records them. */
typedef struct {
  void* start;
  void* kernel_stop;
  void* stop;
} kv_timing_events;

typedef struct {
  float scale;              /* softmax scale; 0 means 1/sqrt(d) ([BT] §07) */
  int32_t partition_tokens; /* split-K partition length in tokens, a positive
                               multiple of B; 0 = the library's choice (one
                               16-token tile for the matrix-core kernel, which
                               rounds a requested length up to whole tiles) */
  int32_t kernel;           /* kv_kernel */
  const kv_timing_events* timing; /* NULL: no timing */
} kv_attention_options;

/* Device workspace needed by paged_attention_decode for these arguments. */
uint64_t paged_attention_workspace_bytes(const kv_pool* pool, int32_t n_seqs, int32_t num_q_heads,
                                         int32_t max_blocks_per_seq,
                                         const kv_attention_options* opts);

/* Decode attention over the paged cache of one layer ([BT] §07): for sequence
 * s with n = context_lens[s] cached tokens (the query's own token included)
 * and query head h reading KV head g = h / (Hq / Hkv),
 *     k_t = K[l][T_s[t / B]][g][t % B],  v_t likewise,   t = 0 .. n-1,
 *     out[s][h] = sum_t softmax_t(scale * q[s][h] . k_t) v_t.
 * The context of every (sequence, kv head) is split into partitions of
 * partition_tokens tokens.  Matrix-core kernel: the partitions of the whole
 * batch are divided evenly, as contiguous runs, among the waves of a
 * persistent grid; a wave folds its consecutive partitions online and writes
 * a running max m, sum l and unnormalised output only where its run of a
 * (sequence, kv head) ends.  Generic kernel: one partial per partition.  A
 * merge kernel folds the partials with the recurrences of [KVM] (chunked
 * prefill mechanism).
 *   q, out:          device [n_seqs][Hq][d], pool dtype (out rounded to
 *                    nearest even for bf16); accumulation is fp32.
 *   d_block_tables:  device int32[n_seqs][max_blocks_per_seq].
 *   d_context_lens:  device int32[n_seqs]; values are clamped to
 *                    max_blocks_per_seq * B; n <= 0 yields a zero row.
 *   d_workspace:     caller-owned device memory of at least
 *                    paged_attention_workspace_bytes, 256-byte aligned (may be
 *                    NULL if that is 0); its contents need no initialisation.
 * A table entry outside [0, N) is never dereferenced: the rows of that
 * sequence are written as NaN.  opts may be NULL (all defaults). */
kv_status paged_attention_decode(kv_pool* pool, int32_t layer, const void* q, void* out,
                                 const int32_t* d_block_tables, const int32_t* d_context_lens,
                                 int32_t n_seqs, int32_t max_blocks_per_seq, int32_t num_q_heads,
                                 const kv_attention_options* opts, void* d_workspace,
                                 uint64_t workspace_bytes, void* hip_stream);

/* paged_attention_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * forbid allocation): the split-K partials live in a static device array the
 * library holds on every GPU it runs on (paged_attention_static_scratch_bytes()
 * bytes, 32 MiB), whose address is looked up on the first call on each device.
 * Nothing is allocated and nothing is cleared; results equal
 * paged_attention_decode's bit for bit.  A call whose workspace
 * (paged_attention_workspace_bytes) would exceed the scratch fails with
 * KV_ERR_INVALID.  Every call on one GPU uses the same scratch, so calls that
 * can overlap on one GPU (on different streams, or from several host threads)
 * race: order them on one stream. */
uint64_t paged_attention_static_scratch_bytes(void);
kv_status paged_attention_decode_static(kv_pool* pool, int32_t layer, const void* q, void* out,
                                        const int32_t* d_block_tables, const int32_t* d_context_lens,
                                        int32_t n_seqs, int32_t max_blocks_per_seq, int32_t num_q_heads,
                                        const kv_attention_options* opts, void* hip_stream);

/* Read-once decode over shared prefixes (cascade).  Sequences are given in
 * groups: group g holds the sequences group_start[g] .. group_start[g+1]-1 (in
 * the order of q, out and the tables), whose tables agree on their first
 * shared_blocks[g] blocks, each completely filled (every member's context is
 * at least 16 * shared_blocks[g] tokens) — forks of one request share such
 * blocks physically ([KVM] CoW branching, cross-turn prefix caching).  The
 * result equals paged_attention_decode; the shared blocks are read once per
 * group instead of once per member.  One persistent kernel streams a single
 * work list of prefix units (a group's shared blocks against the queries of
 * up to 64 query columns -- 32 over a quantised pool, 32 and 16 at d = 256:
 * members x their G heads) and suffix units (a
 * member's remaining blocks against its G heads), cut into per-wave runs by
 * estimated cost; a second kernel folds each member's prefix and suffix
 * partials with the [KVM] recurrences.
 * A member whose shared entries differ from the first member's, or whose
 * context (or the first member's) does not cover them, gets a NaN row (checked
 * on the device); so do the members of a group larger than max_group.  bf16,
 * q8_0 and q4_0 pools (B = 16) with the matrix-core kernel only
 * (KV_ERR_UNSUPPORTED otherwise); over a quantised pool the codes are the
 * matrix operands and the group scales are applied in float32, as in
 * paged_attention_decode ([INF] §8.4.2).
 *   d_group_start:   device int32[n_groups + 1], group_start[0] = 0,
 *                    non-decreasing, group_start[n_groups] = n_seqs.
 *   d_shared_blocks: device int32[n_groups] (0 = no shared prefix).
 *   max_group:       an upper bound of every group's size (sizes the grid).
 *   d_workspace:     paged_attention_cascade_workspace_bytes, 256-byte aligned. */
uint64_t paged_attention_cascade_workspace_bytes(kv_pool* pool, int32_t n_seqs, int32_t n_groups, int32_t max_group,
                                                 int32_t num_q_heads, int32_t max_blocks_per_seq,
                                                 const kv_attention_options* opts);
kv_status paged_attention_decode_cascade(kv_pool* pool, int32_t layer, const void* q, void* out,
                                         const int32_t* d_block_tables, const int32_t* d_context_lens,
                                         int32_t n_seqs, int32_t max_blocks_per_seq, int32_t num_q_heads,
                                         const int32_t* d_group_start, const int32_t* d_shared_blocks,
                                         int32_t n_groups, int32_t max_group, const kv_attention_options* opts,
                                         void* d_workspace, uint64_t workspace_bytes, void* hip_stream);

/* Device workspace needed by paged_attention_prefill for these arguments. */
uint64_t paged_prefill_workspace_bytes(const kv_pool* pool, int32_t n_seqs, int32_t total_q, int32_t max_q_len,
                                       int32_t num_q_heads, int32_t max_blocks_per_seq,
                                       const kv_attention_options* opts);

/* Multi-query attention over the paged cache of one layer: chunked prefill
 * ([KVM] chunked prefill mechanism, Figure 8) and verification of draft
 * positions ([INF] §8.5.1).  Sequence s owns the query rows
 * q_indptr[s] .. q_indptr[s+1]-1, c of them; its K/V rows for those c
 * tokens must already be in the pool (reshape_and_cache), so with
 * n = context_lens[s] the queries sit at positions h = n - c .. n - 1.  The
 * query of chunk row j sees the cached positions 0 .. h + j: the whole
 * history and, inside the chunk, itself and the rows before it.  For query
 * head h reading KV head g = h / (Hq / Hkv):
 *     out[r][h] = sum_{t <= h_s + j} softmax_t(scale * q[r][h] . k_t) v_t.
 * A sequence with c = 1 is a decode query.
 *   q, out:          device [total_q][Hq][d], rows grouped by sequence as
 *                    q_indptr says; bf16 (rounded to nearest even) for bf16
 *                    and quantised pools, f32 for f32 pools.
 *   d_q_indptr:      device int32[n_seqs + 1], non-decreasing, q_indptr[0] = 0,
 *                    q_indptr[n_seqs] <= total_q.  Rows of a sequence that
 *                    would fall outside [0, total_q) are not written.
 *   max_q_len:       an upper bound of every c (sizes the grid); a sequence
 *                    with c > max_q_len or c > n gets NaN rows.
 *   d_block_tables, d_context_lens: as for paged_attention_decode (lengths
 *                    clamped to max_blocks_per_seq * B).
 *   d_workspace:     at least paged_prefill_workspace_bytes, 256-byte
 *                    aligned (NULL if that is 0); no initialisation needed.
 * A table entry outside [0, N) is never dereferenced: every row whose visible
 * keys include it is written as NaN, and so may be the other rows of its
 * query tile (16 consecutive columns of (row, head)) on the multi-query
 * kernels.  Two paths:
 *   multi-query kernels: bf16 pools with B in {4, 8, 16, 32, 64}, d in {64,
 *     128, 256}, and q8_0 / q4_0 pools with B = 16, d in {64, 128}; G <= 16
 *     (KV_KERNEL_AUTO or KV_KERNEL_MFMA); one tile of columns reads each
 *     block once for all its rows.  Over a quantised pool the codes are the
 *     matrix operands (exact in bf16) and the group scales are applied in
 *     float32, as in paged_attention_decode ([INF] §8.4.2);
 *   row-wise: every other pool (f32, quantised at d = 256), and any pool
 *     with KV_KERNEL_GENERIC -- each chunk row is a
 *     decode query over its n - c + j + 1 keys, through the decode kernels
 *     (the matrix-core split-K kernel, in batches of at most 4095 rows, for
 *     quantised pools and bf16 pools of block size 4, 8, 32 or 64; the
 *     generic kernel for f32 pools and other block sizes), so the history is
 *     read once per row.  Rows no sequence owns are written as zero rows.
 *     KV_KERNEL_MFMA on a pool no matrix-core kernel reads gives
 *     KV_ERR_UNSUPPORTED.
 * opts->partition_tokens splits every tile's (row's) keys into partitions
 * merged with the [KVM] recurrences (0 = the library's choice). */
kv_status paged_attention_prefill(kv_pool* pool, int32_t layer, const void* q, void* out,
                                  const int32_t* d_q_indptr, const int32_t* d_block_tables,
                                  const int32_t* d_context_lens, int32_t n_seqs, int32_t total_q,
                                  int32_t max_q_len, int32_t max_blocks_per_seq, int32_t num_q_heads,
                                  const kv_attention_options* opts, void* d_workspace, uint64_t workspace_bytes,
                                  void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
