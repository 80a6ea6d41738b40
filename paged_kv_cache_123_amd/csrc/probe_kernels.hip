// Bandwidth reference: a read-only kernel of known byte count.  It reads a
// buffer as whole 4 KiB blocks (one workgroup of 256 lanes x 16 bytes per
// block) in a caller-given block order, with plain or non-temporal loads, so
// the same access pattern as the paged cache (random 4 KiB blocks) or a
// sequential one can be timed, and hardware byte counters can be calibrated
// against a known size.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pagedkv.h"
#include "status.h"

namespace {

template <bool NT>
__global__ __launch_bounds__(256) void read_blocks_kernel(const uint4* __restrict__ buf,
                                                          const int32_t* __restrict__ order,
                                                          int64_t num_blocks,
                                                          uint32_t* __restrict__ sink) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  uint32_t acc = 0;
  for (int64_t b = blockIdx.x; b < num_blocks; b += gridDim.x) {
    const uint4* p = buf + static_cast<int64_t>(order[b]) * 256 + threadIdx.x;
    uint4 v;
    if constexpr (NT) {
      const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
      v = make_uint4(w.x, w.y, w.z, w.w);
    } else {
      v = *p;
    }
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // a data-dependent store keeps the loads; it practically never fires
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace

extern "C" int32_t pa_probe_read_blocks(const void* buffer, const int32_t* block_order,
                                        int64_t num_blocks, void* sink, int32_t grid,
                                        int32_t non_temporal, void* stream) {
  if (!buffer || !block_order || !sink || num_blocks < 1 || grid < 1)
    return pa::fail(PA_EINVAL, "pa_probe_read_blocks: bad argument");
  if (reinterpret_cast<uintptr_t>(buffer) % 16 != 0)
    return pa::fail(PA_EINVAL, "pa_probe_read_blocks: buffer must be 16-byte aligned");
  if (non_temporal)
    hipLaunchKernelGGL(read_blocks_kernel<true>, dim3(grid), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint4*>(buffer),
                       block_order, num_blocks, static_cast<uint32_t*>(sink));
  else
    hipLaunchKernelGGL(read_blocks_kernel<false>, dim3(grid), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint4*>(buffer),
                       block_order, num_blocks, static_cast<uint32_t*>(sink));
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? PA_OK : pa::fail(PA_ELAUNCH, hipGetErrorString(e));
}
