"""Paged-KV decode path for MI355X (gfx950): hand-written HIP kernels behind
the C ABI of include/pagedkv.h, a C++ host block allocator, and a thin
torch/ctypes binding.

  ops   - compute_slot_mapping, reshape_and_cache, copy_blocks,
          paged_attention_decode, paged_attention_decode_split, the planned,
          multi-query, partials/merge and one-launch step calls
  host  - Pool: the host block allocator (reference counts, copy-on-write)
  step  - DecodeStep: host allocation + one decode step on the device
  cp_step - CPRankStep: one rank's share of a context-parallel step
  session - PagedKVCache: one layer's caches and allocator across many steps
  build - compiles libpagedkv.so in-tree

libpagedkv.so is loaded on first use; every entry point raises ImportError if
it has not been built (there is no fallback path).
"""

from ._lib import PagedKVError, lib

__all__ = ["PagedKVError", "lib"]
