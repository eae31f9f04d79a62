"""Plain, slow CPU oracle for paged single-query decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link
or execute anything in this package: only ``tests/``, ``__graft_entry__.smoke``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library (no headers, kernels, helpers or tables); the only common
dependency is :mod:`synth`, which draws seeded inputs and holds none of the
method's arithmetic.

Sources.  Citations name the pages by title:

* [KVM]  "KV 缓存管理" (KV cache management), chapter 5 of an ML-systems book
         (gptbert.com); its Russian translation "Управление KV-кешем" renders
         some formulas the Chinese extraction garbles.
* [BT]   "KV Cache 还有空间为何新请求却进不来？PagedAttention 的块表与碎片控制"
         (block tables and fragmentation; zwjcode.cn), sections 01-17.
* [INF]  "第 8 章 推理优化" (chapter 8, inference optimization; ai-infra-book).
* [PC]   "第 11 章 KV Cache 内存管理：PagedAttention 与前缀缓存" (shippingwang.com).

Modules:

* :mod:`oracle.footprint`     closed forms: per-token footprint, block bytes,
                               tail waste, reload and recompute times
                               ([KVM] Eq. 1, block-size trade-off,
                               evict-versus-swap analysis; [BT] §01, §04;
                               [INF] §8.1.2, §8.3.1).
* :mod:`oracle.block_manager` the host block manager: FIFO free list,
                               refcounts, tables, append with copy-on-write,
                               fork, release, and the host tier: swap of a
                               sequence's own blocks to pinned host frames and
                               back ([BT] §03-§05, §08, §10, §13; [KVM] paged
                               KV allocation, CoW branching, asynchronous
                               paged swap).
* :mod:`oracle.kv_store`      the logical K/V pool ``[layer][block][slot][head][dim]``
                               ([BT] §06) with slot scatter, block copy and
                               block copies to host frames and back.
* :mod:`oracle.attention`     gathered softmax(q K^T / sqrt(d)) V in float64
                               ([BT] §07) and the split-K merge recurrences
                               ([KVM] chunked prefill mechanism).
* :mod:`oracle.prefill`       multi-query attention over paged history: a chunk
                               of c queries over h cached tokens with the
                               history fully visible and a causal mask inside
                               the chunk ([KVM] chunked prefill mechanism,
                               Figure 8; [INF] §8.2.3 pair counts, §8.5.1
                               verification of draft positions).
* :mod:`oracle.quant`         grouped 8- and 4-bit KV codes with a half scale
                               per 32 values (q8_0, q4_0), their byte budget
                               and read/convert trade-off ([INF] §8.4.2,
                               Figure 8-23), and a quantised logical pool.
* :mod:`oracle.prefix_cache`  radix-tree prefix cache over the block manager:
                               longest match with block-aligned truncation,
                               attach / insert / release, leaf-first LRU
                               eviction ([KVM] cross-turn prefix caching,
                               Table 2, Definition 0.2, estimate 0.4).
* :mod:`oracle.runner`        replays a :mod:`synth` workload through the above.

Every function is pinned by ``tests/test_oracle_pins.py``,
``tests/test_prefill_pins.py``, ``tests/test_quant_pins.py``,
``tests/test_prefix_cache.py`` and ``tests/test_swap_pins.py`` against values the
pages print, closed forms, invariants and brute force.  Parity unpinned: none.
"""
