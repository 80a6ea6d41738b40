// Integer and copy kernels of the paged-KV path: slot mapping, the cache
// scatter of new tokens, and whole-block copies for copy-on-write.
//
// Sources: [PUFANYI] "按 Block 分配" (position -> logical block -> physical
// block + offset); [CSDN] section 2.3 (per-request slot mapping over
// query_start_loc); [VLLBC] paper sections 4.2 and 4.4 / Fig. 8 (new tokens
// fill the tail block; copy-on-write copies one whole block).
//
// All three are bandwidth-trivial; they move 16-byte units per lane so every
// wave touches whole 1 KiB runs of the cache.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "launch.h"

namespace pa {
namespace {

// Slot of one token position under one table row ([PUFANYI] "按 Block 分配":
// logical block pos / B, physical block row[pos / B], offset pos % B).
//
// Context parallelism ([CSDN] section 2.3 describes the placement): the
// ranks of a group share a table whose entries name virtual blocks of
// B * cp_world positions.  Inside a virtual block, runs of `interleave`
// consecutive positions are dealt to the ranks in turn; a rank keeps its
// runs in order, so its k-th run fills local offsets [k * interleave,
// (k + 1) * interleave) of the block with the same number in its own cache.
// Positions dealt to another rank give -1.  cp_world = interleave = 1 is the
// plain mapping.
__device__ __forceinline__ int64_t slot_of(const int32_t* __restrict__ row, int64_t pos,
                                           int32_t block_size, int32_t cp_world,
                                           int32_t cp_rank, int32_t interleave) {
  const int64_t span = static_cast<int64_t>(block_size) * cp_world;
  const int64_t vblock = pos / span;
  const int64_t within = pos - vblock * span;
  const int64_t run = within / interleave;  // index of the run inside the block
  if (run % cp_world != cp_rank) return -1;
  const int64_t local = (run / cp_world) * interleave + (within - run * interleave);
  return static_cast<int64_t>(row[vblock]) * block_size + local;
}

// One thread per entry of slot_mapping[0, max_num_tokens).  Token i <
// num_tokens belongs to the last request r with qsl[r] <= i (a binary search
// over the request offsets, so empty requests are skipped); entries from
// num_tokens on are padding and get -1.
__global__ __launch_bounds__(256) void slot_mapping_kernel(
    const int32_t* __restrict__ qsl, const int64_t* __restrict__ positions,
    const int32_t* __restrict__ block_tables, int64_t bt_stride, int32_t num_reqs,
    int64_t num_tokens, int64_t max_num_tokens, int32_t block_size, int32_t cp_world,
    int32_t cp_rank, int32_t interleave, int64_t* __restrict__ slot_mapping) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= max_num_tokens) return;
  if (i >= num_tokens) {
    slot_mapping[i] = -1;
    return;
  }
  int32_t lo = 0, hi = num_reqs;  // invariant: qsl[lo] <= i < qsl[hi]
  while (hi - lo > 1) {
    const int32_t mid = lo + (hi - lo) / 2;
    if (qsl[mid] <= i) lo = mid; else hi = mid;
  }
  slot_mapping[i] = slot_of(block_tables + static_cast<int64_t>(lo) * bt_stride, positions[i],
                            block_size, cp_world, cp_rank, interleave);
}

// One workgroup per token.  Unit = 16 bytes when every row start is 16-byte
// aligned, else the element size; the copy is a bit copy either way.
template <typename U>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const U* __restrict__ key, const U* __restrict__ value, int64_t key_stride_u,
    int64_t value_stride_u, U* __restrict__ key_cache, U* __restrict__ value_cache,
    const int64_t* __restrict__ slot_mapping, int32_t row_units, int32_t head_units,
    int32_t block_size) {
  const int64_t i = blockIdx.x;
  const int64_t slot = slot_mapping[i];
  if (slot < 0) return;
  const int64_t blk = slot / block_size;
  const int64_t off = slot % block_size;
  const int32_t num_heads = row_units / head_units;
  const U* ksrc = key + i * key_stride_u;
  const U* vsrc = value + i * value_stride_u;
  // cache element (blk, h, off, :) starts at ((blk * H + h) * B + off) * head
  for (int32_t u = threadIdx.x; u < row_units; u += blockDim.x) {
    const int32_t h = u / head_units, e = u % head_units;
    const int64_t dst = ((blk * num_heads + h) * block_size + off) * head_units + e;
    key_cache[dst] = ksrc[u];
    value_cache[dst] = vsrc[u];
  }
}

// grid.x = pair, grid.y = chunk of the block; a block is one contiguous run of
// block_units 16-byte units in each cache.
__global__ __launch_bounds__(256) void copy_blocks_kernel(
    uint4* __restrict__ key_cache, uint4* __restrict__ value_cache,
    const int64_t* __restrict__ block_mapping, int64_t block_units, int64_t chunk_units) {
  const int64_t pair = blockIdx.x;
  const int64_t src = block_mapping[2 * pair], dst = block_mapping[2 * pair + 1];
  const int64_t begin = blockIdx.y * chunk_units;
  const int64_t end = begin + chunk_units < block_units ? begin + chunk_units : block_units;
  const uint4* ks = key_cache + src * block_units;
  const uint4* vs = value_cache + src * block_units;
  uint4* kd = key_cache + dst * block_units;
  uint4* vd = value_cache + dst * block_units;
  for (int64_t u = begin + threadIdx.x; u < end; u += blockDim.x) {
    kd[u] = ks[u];
    vd[u] = vs[u];
  }
}

// Table validation: result[0] counts the sequences whose length or table
// entries are invalid, result[1] receives the smallest such sequence (or
// INT32_MAX when none).  The entries read are only those the attention reads
// (blocks [lo / B, ceil(L / B)), lo the window start), after the row width is
// checked, so a bad length is reported rather than followed.
__global__ void validate_init_kernel(int32_t* __restrict__ result) {
  if (threadIdx.x == 0) {
    result[0] = 0;
    result[1] = INT32_MAX;
  }
}

__global__ __launch_bounds__(256) void validate_tables_kernel(
    const int32_t* __restrict__ block_tables, int64_t bt_stride,
    const int32_t* __restrict__ context_lens, int32_t block_size, int32_t num_blocks,
    int32_t window, int32_t* __restrict__ result) {
  __shared__ int bad;
  const int32_t s = blockIdx.x;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  const int64_t L = context_lens[s];
  const int64_t nb = (L + block_size - 1) / block_size;
  if (L < 0 || nb > bt_stride) {
    if (threadIdx.x == 0) bad = 1;
  } else {
    const int64_t lo = window > 0 ? (L - window > 0 ? L - window : 0) : 0;
    const int32_t* row = block_tables + static_cast<int64_t>(s) * bt_stride;
    for (int64_t j = lo / block_size + threadIdx.x; j < nb; j += blockDim.x) {
      const int32_t b = row[j];
      if (b < 0 || b >= num_blocks) bad = 1;  // benign race: every writer stores 1
    }
  }
  __syncthreads();
  if (threadIdx.x == 0 && bad) {
    atomicAdd(&result[0], 1);
    atomicMin(&result[1], s);
  }
}

}  // namespace

hipError_t launch_slot_mapping(const int32_t* query_start_loc, const int64_t* positions,
                               const int32_t* block_tables, int64_t bt_stride, int32_t num_reqs,
                               int64_t num_tokens, int64_t max_num_tokens, int32_t block_size,
                               int32_t cp_world, int32_t cp_rank, int32_t interleave,
                               int64_t* slot_mapping, hipStream_t stream) {
  if (max_num_tokens == 0) return hipSuccess;
  const int64_t grid = (max_num_tokens + 255) / 256;
  hipLaunchKernelGGL(slot_mapping_kernel, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream,
                     query_start_loc, positions, block_tables, bt_stride, num_reqs, num_tokens,
                     max_num_tokens, block_size, cp_world, cp_rank, interleave, slot_mapping);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache(const void* key, const void* value, int64_t key_stride,
                                    int64_t value_stride, void* key_cache, void* value_cache,
                                    const int64_t* slot_mapping, int64_t num_tokens,
                                    int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                                    int32_t elem_bytes, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int64_t head_bytes = static_cast<int64_t>(head_size) * elem_bytes;
  const bool vec16 = head_bytes % 16 == 0 && (key_stride * elem_bytes) % 16 == 0 &&
                     (value_stride * elem_bytes) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(key) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(value) % 16 == 0;
  const dim3 grid(static_cast<uint32_t>(num_tokens));
  if (vec16) {
    const int32_t head_units = static_cast<int32_t>(head_bytes / 16);
    const int32_t row_units = head_units * num_kv_heads;
    const int32_t threads = row_units < 256 ? ((row_units + 63) / 64) * 64 : 256;
    hipLaunchKernelGGL(reshape_and_cache_kernel<uint4>, grid, dim3(threads), 0, stream,
                       static_cast<const uint4*>(key), static_cast<const uint4*>(value),
                       key_stride * elem_bytes / 16, value_stride * elem_bytes / 16,
                       static_cast<uint4*>(key_cache), static_cast<uint4*>(value_cache),
                       slot_mapping, row_units, head_units, block_size);
  } else if (elem_bytes == 4) {
    const int32_t row_units = head_size * num_kv_heads;
    hipLaunchKernelGGL(reshape_and_cache_kernel<uint32_t>, grid, dim3(256), 0, stream,
                       static_cast<const uint32_t*>(key), static_cast<const uint32_t*>(value),
                       key_stride, value_stride, static_cast<uint32_t*>(key_cache),
                       static_cast<uint32_t*>(value_cache), slot_mapping, row_units, head_size,
                       block_size);
  } else {
    const int32_t row_units = head_size * num_kv_heads;
    hipLaunchKernelGGL(reshape_and_cache_kernel<uint16_t>, grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(key), static_cast<const uint16_t*>(value),
                       key_stride, value_stride, static_cast<uint16_t*>(key_cache),
                       static_cast<uint16_t*>(value_cache), slot_mapping, row_units, head_size,
                       block_size);
  }
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* key_cache, void* value_cache, const int64_t* block_mapping,
                              int64_t num_pairs, int64_t block_bytes, hipStream_t stream) {
  if (num_pairs == 0) return hipSuccess;
  const int64_t block_units = block_bytes / 16;
  const int64_t chunk_units = 2048;  // 32 KiB of each cache per workgroup
  const int64_t chunks = (block_units + chunk_units - 1) / chunk_units;
  hipLaunchKernelGGL(copy_blocks_kernel,
                     dim3(static_cast<uint32_t>(num_pairs), static_cast<uint32_t>(chunks)),
                     dim3(256), 0, stream, static_cast<uint4*>(key_cache),
                     static_cast<uint4*>(value_cache), block_mapping, block_units, chunk_units);
  return hipGetLastError();
}

hipError_t launch_validate_tables(const int32_t* block_tables, int64_t bt_stride,
                                  const int32_t* context_lens, int32_t num_seqs,
                                  int32_t block_size, int32_t num_blocks, int32_t window,
                                  int32_t* result, hipStream_t stream) {
  hipLaunchKernelGGL(validate_init_kernel, dim3(1), dim3(64), 0, stream, result);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(validate_tables_kernel, dim3(static_cast<uint32_t>(num_seqs)), dim3(256), 0,
                     stream, block_tables, bt_stride, context_lens, block_size, num_blocks,
                     window, result);
  return hipGetLastError();
}

}  // namespace pa

