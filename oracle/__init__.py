"""CPU oracle for the paged-KV decode path — TEST INFRASTRUCTURE, not product.

A plain, slow, obviously-correct restatement of what the paged KV cache
computes, written from the four web pages on PagedAttention:

  [CSDN]   "PagedAttention 核心创新深度分析" (openeuler.csdn.net), sections
           2.3 (BlockTable / slot-mapping), 2.4 (BlockPool), 3.1.2 (free),
           3.2.1 (get_new_blocks), 3.2.3 (touch), 3.2.4 (free_blocks).
  [VLLBC]  "paged-attention-kv-cache" visual reading (blog.vllbc.top): the
           walk-through of paper §4.2, §4.4 / Fig. 8, the sharing simulator,
           and the §7.2 tail-fragmentation example.
  [DEEPSONAR] "vLLM 的 PagedAttention：显存管理如何撑起大模型推理"
           (deepsonar.com.cn), sections 2.1-2.3, 2.6 and 七.
  [PUFANYI] "Infra: PagedAttention" (pufanyi.com), sections "按 Block 分配"
           and "共享前缀，分叉时 Copy-on-write".

Floating point is evaluated in float64.  Storage dtypes are decoded exactly
(bf16 bits << 16 -> fp32 -> fp64; fp16 -> fp64; fp32 -> fp64).

Who may use this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``.  The product library never imports it,
and it imports nothing from the product (``paged_kv_cache_123_amd``).

Parity status per function (what pins it is listed in each module header):
  allocator.OraclePool ................ pinned (worked examples of the pages)
  slots.compute_slot_mapping .......... pinned (table [3,0,4] example, growth
                                        example, bijection invariants)
  cache_ops.reshape_and_cache/copy_blocks  pinned (round-trip invariants)
  attention.paged_attention ........... pinned (library softmax brute force,
                                        closed forms, invariances)
  attention.split_partials/merge ...... pinned (equality with single pass)
  attention.paged_attention_multi ..... pinned (dense causal softmax)
  slots.compute_slot_mapping_cp,
  slots.cp_local_length ............... pinned (hand-computed interleaves, world
                                        1 = plain mapping, every position on
                                        one rank, local offsets in order)
  attention.paged_attention_partials,
  attention.merge_rank_partials ....... pinned (rank shares merge to dense
                                        softmax attention; share partial =
                                        partial over the owned positions)
  slots.map_to_kernel_blocks .......... pinned (the [0,1,2] x 2 example; slots
                                        agree under both block sizes)
  attention.* with window > 0,
  allocator.OraclePool.remove_skipped . pinned (banded dense softmax, closed
                                        forms, released blocks never read)
  prefix_cache.* ...................... pinned (FIPS 180 digests, chaining,
                                        first-miss stop, n - 1 cap, full
                                        blocks only, LRU eviction, touch)
  dtypes.decode ....................... pinned (bit patterns with known values)
"""

from . import allocator, attention, cache_ops, dtypes, prefix_cache, slots  # noqa: F401

__all__ = ["allocator", "attention", "cache_ops", "dtypes", "prefix_cache", "slots"]
