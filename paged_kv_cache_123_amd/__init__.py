"""Paged-KV decode path for MI355X (gfx950): hand-written HIP kernels behind
the C ABI of include/pagedkv.h, a C++ host block allocator, and a thin
torch/ctypes binding.

  ops   - compute_slot_mapping, reshape_and_cache, copy_blocks,
          paged_attention_decode, paged_attention_decode_split
  host  - Pool: the host block allocator (reference counts, copy-on-write)
  step  - DecodeStep: host allocation + one decode step on the device

Importing the package loads libpagedkv.so and raises if it is not built.
"""

from ._lib import PagedKVError, lib

lib()  # fail loudly when the HIP library has not been built

__all__ = ["PagedKVError", "lib"]
