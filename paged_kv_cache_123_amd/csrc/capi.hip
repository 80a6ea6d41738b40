// extern "C" entry points of the device half of pagedkv.h: host-side argument
// validation, then the launch on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <string>

#include "launch.h"
#include "pagedkv.h"
#include "status.h"

namespace {

using pa::fail;

int32_t elem_bytes(int32_t dtype) {
  switch (dtype) {
    case PA_F32: return 4;
    case PA_F16: return 2;
    case PA_BF16: return 2;
    default: return 0;
  }
}

bool pow2_in(int32_t v, int32_t lo, int32_t hi) {
  return v >= lo && v <= hi && (v & (v - 1)) == 0;
}

bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

int32_t launched(hipError_t e, const char* who) {
  if (e == hipSuccess) return PA_OK;
  std::string msg = std::string(who) + ": launch failed: " + hipGetErrorString(e);
  return fail(PA_ELAUNCH, msg.c_str());
}

// Shared checks of the two attention entry points.
int32_t check_decode(const char* who, void* out, const void* query, const void* key_cache,
                     const void* value_cache, const int32_t* block_tables, int64_t bt_stride,
                     const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                     int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                     int32_t max_context_len, int32_t dtype) {
  std::string w(who);
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens)
    return fail(PA_EINVAL, (w + ": NULL pointer").c_str());
  if (num_seqs < 1 || num_heads < 1 || num_kv_heads < 1 || max_context_len < 1)
    return fail(PA_EINVAL, (w + ": sizes must be >= 1").c_str());
  if (num_heads % num_kv_heads != 0)
    return fail(PA_EINVAL, (w + ": num_heads must be a multiple of num_kv_heads").c_str());
  const int32_t g = num_heads / num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8)
    return fail(PA_EINVAL, (w + ": num_heads / num_kv_heads must be 1, 2, 4 or 8").c_str());
  if (head_size != 64 && head_size != 128)
    return fail(PA_EINVAL, (w + ": head_size must be 64 or 128").c_str());
  if (!pow2_in(block_size, 1, 128))
    return fail(PA_EINVAL, (w + ": block_size must be a power of two in [1, 128]").c_str());
  if (elem_bytes(dtype) == 0) return fail(PA_EINVAL, (w + ": unknown dtype").c_str());
  if (bt_stride < (max_context_len + block_size - 1) / block_size)
    return fail(PA_EINVAL, (w + ": bt_stride smaller than ceil(max_context_len / B)").c_str());
  if (!aligned16(out) || !aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache))
    return fail(PA_EINVAL, (w + ": out, query and caches must be 16-byte aligned").c_str());
  // every grid is one-dimensional: (sequence, KV head) workgroups of a
  // launch without a work list, (sequence, four heads) of the merge
  if (static_cast<int64_t>(num_seqs) * num_kv_heads > INT32_MAX ||
      static_cast<int64_t>(num_seqs) * ((num_heads + 3) / 4) > INT32_MAX)
    return fail(PA_EINVAL, (w + ": num_seqs x heads exceeds one launch's workgroups").c_str());
  return PA_OK;
}

// A split launch without a work list has a workgroup per (sequence, KV head,
// partition), whether the partition holds tokens or not.
int32_t check_split_grid(const char* who, int32_t num_seqs, int32_t num_kv_heads,
                         int32_t max_context_len, int32_t partition_size) {
  const int64_t np = (static_cast<int64_t>(max_context_len) + partition_size - 1) / partition_size;
  if (np * num_kv_heads * num_seqs > INT32_MAX)
    return fail(PA_EINVAL, (std::string(who) + ": num_seqs x num_kv_heads x partitions exceeds "
                            "one launch's workgroups")
                               .c_str());
  return PA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Sections of a split workspace: max_logits and exp_sums [rows][H][NP], then
// tmp_out [rows][H][NP][D], each starting on a 256-byte boundary.
struct SplitLayout {
  int32_t np;
  size_t sum_off, out_off, bytes;
};

SplitLayout split_layout(int64_t rows, int32_t num_heads, int32_t head_size,
                         int32_t max_context_len, int32_t partition_size) {
  SplitLayout w{};
  w.np = (max_context_len + partition_size - 1) / partition_size;
  const size_t parts = static_cast<size_t>(rows) * num_heads * w.np;
  w.sum_off = align256(parts * sizeof(float));
  w.out_off = 2 * w.sum_off;
  w.bytes = w.out_off + align256(parts * head_size * sizeof(float));
  return w;
}

// Points the launch arguments at the sections of a checked workspace.
void set_split(pa::DecodeArgs& a, void* workspace, const SplitLayout& w, int32_t partition_size) {
  char* ws = static_cast<char*>(workspace);
  a.partition_size = partition_size;
  a.num_partitions = w.np;
  a.ws_max = reinterpret_cast<float*>(ws);
  a.ws_sum = reinterpret_cast<float*>(ws + w.sum_off);
  a.ws_out = reinterpret_cast<float*>(ws + w.out_off);
}

// Every new token of a sequence is a query: the query vectors of one work item
// (max_query_len x heads per KV head) must fit one workgroup.
int32_t check_query_capacity(const char* who, int32_t max_query_len, int32_t num_heads,
                             int32_t num_kv_heads, int32_t head_size, int32_t dtype) {
  if (max_query_len < 1)
    return fail(PA_EINVAL, (std::string(who) + ": max_query_len must be >= 1").c_str());
  const int64_t nq = static_cast<int64_t>(max_query_len) * (num_heads / num_kv_heads);
  const bool matrix = (dtype == PA_F16 || dtype == PA_BF16) && head_size == 128;
  if (nq > (matrix ? 16 : 8))
    return fail(PA_EINVAL, (std::string(who) + ": max_query_len x (num_heads / num_kv_heads) "
                            "must be at most 16 (16-bit storage, head_size 128) or 8")
                               .c_str());
  return PA_OK;
}

// Split-K workspace of pa_paged_attention_decode_split_noalloc: a static
// device array, so that launch needs no allocation.  Each GPU the library
// runs on holds its own copy until the process ends.  Host code never passes
// the array's name to a kernel (on the host it is only a stand-in): the
// device address of the current GPU's copy is looked up once per device
// with hipGetSymbolAddress and kept here.
static __device__ __align__(256) char scratch[PA_NOALLOC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

int32_t noalloc_workspace(const char* who, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return launched(e, who);
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PA_EINVAL, (std::string(who) + ": device index beyond 63").c_str());
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return launched(e != hipSuccess ? e : hipErrorInvalidSymbol, who);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

extern "C" {

int32_t pa_compute_slot_mapping(const int32_t* query_start_loc, const int64_t* positions,
                                const int32_t* block_tables, int64_t bt_stride,
                                int32_t num_reqs, int64_t num_tokens, int64_t max_num_tokens,
                                int32_t block_size, int64_t* slot_mapping, void* stream) {
  if (!query_start_loc || !block_tables || !slot_mapping || (!positions && num_tokens > 0))
    return fail(PA_EINVAL, "pa_compute_slot_mapping: NULL pointer");
  if (num_reqs < 1 || num_tokens < 0 || max_num_tokens < num_tokens ||
      max_num_tokens > INT32_MAX || bt_stride < 1 || block_size < 1)
    return fail(PA_EINVAL, "pa_compute_slot_mapping: bad sizes");
  return launched(pa::launch_slot_mapping(query_start_loc, positions, block_tables, bt_stride,
                                          num_reqs, num_tokens, max_num_tokens, block_size, 1, 0,
                                          1, slot_mapping, static_cast<hipStream_t>(stream)),
                  "pa_compute_slot_mapping");
}

int32_t pa_compute_slot_mapping_cp(const int32_t* query_start_loc, const int64_t* positions,
                                   const int32_t* block_tables, int64_t bt_stride,
                                   int32_t num_reqs, int64_t num_tokens, int64_t max_num_tokens,
                                   int32_t block_size, int32_t cp_world, int32_t cp_rank,
                                   int32_t interleave, int64_t* slot_mapping, void* stream) {
  const char* who = "pa_compute_slot_mapping_cp";
  if (!query_start_loc || !block_tables || !slot_mapping || (!positions && num_tokens > 0))
    return fail(PA_EINVAL, "pa_compute_slot_mapping_cp: NULL pointer");
  if (num_reqs < 1 || num_tokens < 0 || max_num_tokens < num_tokens ||
      max_num_tokens > INT32_MAX || bt_stride < 1 || block_size < 1)
    return fail(PA_EINVAL, "pa_compute_slot_mapping_cp: bad sizes");
  if (cp_world < 1 || cp_rank < 0 || cp_rank >= cp_world)
    return fail(PA_EINVAL, "pa_compute_slot_mapping_cp: need 0 <= cp_rank < cp_world");
  if (interleave < 1 || block_size % interleave != 0)
    return fail(PA_EINVAL, "pa_compute_slot_mapping_cp: interleave must divide block_size");
  return launched(pa::launch_slot_mapping(query_start_loc, positions, block_tables, bt_stride,
                                          num_reqs, num_tokens, max_num_tokens, block_size,
                                          cp_world, cp_rank, interleave, slot_mapping,
                                          static_cast<hipStream_t>(stream)),
                  who);
}

int32_t pa_reshape_and_cache(const void* key, const void* value, int64_t key_stride,
                             int64_t value_stride, void* key_cache, void* value_cache,
                             const int64_t* slot_mapping, int64_t num_tokens,
                             int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                             int32_t dtype, void* stream) {
  const int32_t eb = elem_bytes(dtype);
  if (eb == 0) return fail(PA_EINVAL, "pa_reshape_and_cache: unknown dtype");
  if (num_tokens < 0 || num_kv_heads < 1 || head_size < 1 || block_size < 1)
    return fail(PA_EINVAL, "pa_reshape_and_cache: bad sizes");
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping)
    return fail(PA_EINVAL, "pa_reshape_and_cache: NULL pointer");
  const int64_t row = static_cast<int64_t>(num_kv_heads) * head_size;
  if (key_stride < row || value_stride < row)
    return fail(PA_EINVAL, "pa_reshape_and_cache: stride smaller than num_kv_heads*head_size");
  if (!aligned16(key_cache) || !aligned16(value_cache))
    return fail(PA_EINVAL, "pa_reshape_and_cache: caches must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(key) % eb != 0 || reinterpret_cast<uintptr_t>(value) % eb != 0)
    return fail(PA_EINVAL, "pa_reshape_and_cache: key/value not aligned to their element size");
  return launched(pa::launch_reshape_and_cache(key, value, key_stride, value_stride, key_cache,
                                               value_cache, slot_mapping, num_tokens,
                                               num_kv_heads, head_size, block_size, eb,
                                               static_cast<hipStream_t>(stream)),
                  "pa_reshape_and_cache");
}

int32_t pa_copy_blocks(void* key_cache, void* value_cache, const int64_t* block_mapping,
                       int64_t num_pairs, int32_t num_kv_heads, int32_t head_size,
                       int32_t block_size, int32_t dtype, void* stream) {
  const int32_t eb = elem_bytes(dtype);
  if (eb == 0) return fail(PA_EINVAL, "pa_copy_blocks: unknown dtype");
  if (num_pairs < 0 || num_kv_heads < 1 || head_size < 1 || block_size < 1)
    return fail(PA_EINVAL, "pa_copy_blocks: bad sizes");
  if (num_pairs == 0) return PA_OK;
  if (!key_cache || !value_cache || !block_mapping)
    return fail(PA_EINVAL, "pa_copy_blocks: NULL pointer");
  const int64_t block_bytes =
      static_cast<int64_t>(num_kv_heads) * block_size * head_size * eb;
  if (block_bytes % 16 != 0 || !aligned16(key_cache) || !aligned16(value_cache))
    return fail(PA_EINVAL, "pa_copy_blocks: blocks must be whole 16-byte units, caches aligned");
  return launched(pa::launch_copy_blocks(key_cache, value_cache, block_mapping, num_pairs,
                                         block_bytes, static_cast<hipStream_t>(stream)),
                  "pa_copy_blocks");
}

int32_t pa_paged_attention_decode(void* out, const void* query, const void* key_cache,
                                  const void* value_cache, const int32_t* block_tables,
                                  int64_t bt_stride, const int32_t* context_lens,
                                  int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                  int32_t head_size, int32_t block_size,
                                  int32_t max_context_len, float scale, int32_t dtype,
                                  void* stream) {
  int32_t st = check_decode("pa_paged_attention_decode", out, query, key_cache, value_cache,
                            block_tables, bt_stride, context_lens, num_seqs, num_heads,
                            num_kv_heads, head_size, block_size, max_context_len, dtype);
  if (st != PA_OK) return st;
  pa::DecodeArgs a{out, query, key_cache, value_cache, block_tables, bt_stride, context_lens,
                   num_seqs, num_heads, num_kv_heads, head_size, block_size,
                   /*partition_size=*/0, /*num_partitions=*/1, scale, dtype,
                   nullptr, nullptr, nullptr, nullptr, 0};
  return launched(pa::launch_decode(a, static_cast<hipStream_t>(stream)),
                  "pa_paged_attention_decode");
}

int32_t pa_set_decode_kernel(int32_t mode) {
  if (mode < 0 || mode > 2) {
    fail(PA_EINVAL, "pa_set_decode_kernel: mode must be 0, 1 or 2");
    return -1;
  }
  return pa::set_decode_kernel(mode);
}

size_t pa_split_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_size,
                                int32_t max_context_len, int32_t partition_size) {
  if (num_seqs < 1 || num_heads < 1 || head_size < 1 || max_context_len < 1 ||
      partition_size < 1)
    return 0;
  return split_layout(num_seqs, num_heads, head_size, max_context_len, partition_size).bytes;
}

int32_t pa_split_workspace_layout(int32_t num_seqs, int32_t num_heads, int32_t head_size,
                                  int32_t max_context_len, int32_t partition_size,
                                  int64_t* offsets_out, int32_t* num_partitions_out) {
  if (!offsets_out || !num_partitions_out || num_seqs < 1 || num_heads < 1 || head_size < 1 ||
      max_context_len < 1 || partition_size < 1)
    return fail(PA_EINVAL, "pa_split_workspace_layout: bad argument");
  const SplitLayout w =
      split_layout(num_seqs, num_heads, head_size, max_context_len, partition_size);
  offsets_out[0] = 0;
  offsets_out[1] = static_cast<int64_t>(w.sum_off);
  offsets_out[2] = static_cast<int64_t>(w.out_off);
  *num_partitions_out = w.np;
  return PA_OK;
}

static int32_t decode_split_impl(const char* who, void* out, const void* query,
                                 const void* key_cache, const void* value_cache,
                                 const int32_t* block_tables, int64_t bt_stride,
                                 const int32_t* context_lens, int32_t num_seqs,
                                 int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                                 int32_t block_size, int32_t max_context_len, float scale,
                                 int32_t dtype, int32_t partition_size, void* workspace,
                                 size_t workspace_bytes, bool static_workspace, void* stream) {
  const std::string w(who);
  int32_t st = check_decode(who, out, query, key_cache, value_cache, block_tables, bt_stride,
                            context_lens, num_seqs, num_heads, num_kv_heads, head_size,
                            block_size, max_context_len, dtype);
  if (st != PA_OK) return st;
  if (partition_size < 16 || partition_size > 4096 || partition_size % 16 != 0 ||
      partition_size % block_size != 0)
    return fail(PA_EINVAL, (w + ": partition_size must be a multiple of 16 and of block_size, "
                                "at most 4096").c_str());
  const size_t need = pa_split_workspace_bytes(num_seqs, num_heads, head_size, max_context_len,
                                               partition_size);
  if (static_workspace) {
    if (need > PA_NOALLOC_WORKSPACE_BYTES)
      return fail(PA_EINVAL, (w + ": the split workspace of this launch exceeds the library's "
                                  "static PA_NOALLOC_WORKSPACE_BYTES").c_str());
  } else {
    if (!workspace || workspace_bytes < need)
      return fail(PA_EINVAL, (w + ": workspace missing or too small").c_str());
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
      return fail(PA_EINVAL, (w + ": workspace must be 256-byte aligned").c_str());
  }
  st = check_split_grid(who, num_seqs, num_kv_heads, max_context_len, partition_size);
  if (st != PA_OK) return st;
  if (static_workspace) {  // every host check passed: now the device's array
    st = noalloc_workspace(who, &workspace);
    if (st != PA_OK) return st;
  }
  pa::DecodeArgs a{out, query, key_cache, value_cache, block_tables, bt_stride, context_lens,
                   num_seqs, num_heads, num_kv_heads, head_size, block_size, 0, 1, scale,
                   dtype, nullptr, nullptr, nullptr, nullptr, 0};
  set_split(a, workspace,
            split_layout(num_seqs, num_heads, head_size, max_context_len, partition_size),
            partition_size);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  st = launched(pa::launch_decode(a, s), (w + " (partition)").c_str());
  if (st != PA_OK) return st;
  return launched(pa::launch_split_reduce(a, s), (w + " (reduce)").c_str());
}

int32_t pa_paged_attention_decode_split(void* out, const void* query, const void* key_cache,
                                        const void* value_cache, const int32_t* block_tables,
                                        int64_t bt_stride, const int32_t* context_lens,
                                        int32_t num_seqs, int32_t num_heads,
                                        int32_t num_kv_heads, int32_t head_size,
                                        int32_t block_size, int32_t max_context_len,
                                        float scale, int32_t dtype, int32_t partition_size,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  return decode_split_impl("pa_paged_attention_decode_split", out, query, key_cache, value_cache,
                           block_tables, bt_stride, context_lens, num_seqs, num_heads,
                           num_kv_heads, head_size, block_size, max_context_len, scale, dtype,
                           partition_size, workspace, workspace_bytes, false, stream);
}

int32_t pa_paged_attention_decode_split_noalloc(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, int64_t bt_stride, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
    int32_t block_size, int32_t max_context_len, float scale, int32_t dtype,
    int32_t partition_size, void* stream) {
  return decode_split_impl("pa_paged_attention_decode_split_noalloc", out, query, key_cache,
                           value_cache, block_tables, bt_stride, context_lens, num_seqs,
                           num_heads, num_kv_heads, head_size, block_size, max_context_len, scale,
                           dtype, partition_size, nullptr, 0, true, stream);
}

int32_t pa_paged_attention_decode_planned(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, int64_t bt_stride, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
    int32_t block_size, int32_t max_context_len, float scale, int32_t dtype,
    int32_t partition_size, const int32_t* work_items, int64_t num_work_items,
    const int32_t* shared_prefix_blocks, void* workspace, size_t workspace_bytes,
    int32_t sliding_window, void* stream) {
  const char* who = "pa_paged_attention_decode_planned";
  if (sliding_window < 0)
    return fail(PA_EINVAL, "pa_paged_attention_decode_planned: sliding_window < 0");
  int32_t st = check_decode(who, out, query, key_cache, value_cache, block_tables, bt_stride,
                            context_lens, num_seqs, num_heads, num_kv_heads, head_size,
                            block_size, max_context_len, dtype);
  if (st != PA_OK) return st;
  if (!work_items || num_work_items < 1 ||
      num_work_items > static_cast<int64_t>(0x7fffffff) / num_kv_heads)
    return fail(PA_EINVAL, "pa_paged_attention_decode_planned: bad work list");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (partition_size == 0) {
    pa::DecodeArgs a{out, query, key_cache, value_cache, block_tables, bt_stride, context_lens,
                     num_seqs, num_heads, num_kv_heads, head_size, block_size, 0, 1, scale,
                     dtype, nullptr, nullptr, nullptr, work_items, num_work_items};
    a.shared_blocks = shared_prefix_blocks;
    a.window = sliding_window;
    return launched(pa::launch_decode(a, s), who);
  }
  if (partition_size < 16 || partition_size > 4096 || partition_size % 16 != 0 ||
      partition_size % block_size != 0)
    return fail(PA_EINVAL,
                "pa_paged_attention_decode_planned: partition_size must be 0, or a multiple of "
                "16 and of block_size, at most 4096");
  const size_t need = pa_split_workspace_bytes(num_seqs, num_heads, head_size, max_context_len,
                                               partition_size);
  if (!workspace || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(PA_EINVAL,
                "pa_paged_attention_decode_planned: workspace missing, too small or misaligned");
  pa::DecodeArgs a{out, query, key_cache, value_cache, block_tables, bt_stride, context_lens,
                   num_seqs, num_heads, num_kv_heads, head_size, block_size, 0, 1, scale, dtype,
                   nullptr, nullptr, nullptr, work_items, num_work_items};
  set_split(a, workspace,
            split_layout(num_seqs, num_heads, head_size, max_context_len, partition_size),
            partition_size);
  a.shared_blocks = shared_prefix_blocks;
  a.window = sliding_window;
  st = launched(pa::launch_decode(a, s), "pa_paged_attention_decode_planned (partition)");
  if (st != PA_OK) return st;
  return launched(pa::launch_split_reduce(a, s), "pa_paged_attention_decode_planned (reduce)");
}

static int32_t decode_step_impl(const char* who, int32_t max_group, bool chunked, void* out,
                                const void* query, void* key_cache, void* value_cache,
                                const int32_t* block_tables, int64_t bt_stride,
                                const int32_t* context_lens, int32_t num_seqs,
                                int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                                int32_t block_size, int32_t max_context_len, float scale,
                                int32_t dtype, int32_t partition_size,
                                const int32_t* work_items, int64_t num_work_items,
                                const int32_t* shared_prefix_blocks, void* workspace,
                                size_t workspace_bytes, const int32_t* query_start_loc,
                                const void* key, const void* value, int64_t key_stride,
                                int64_t value_stride, const int64_t* cow_src,
                                int64_t* slot_mapping, int32_t max_query_len,
                                int32_t sliding_window, void* stream) {
  if (sliding_window < 0)
    return fail(PA_EINVAL, (std::string(who) + ": sliding_window < 0").c_str());
  int32_t st = check_decode(who, out, query, key_cache, value_cache, block_tables, bt_stride,
                            context_lens, num_seqs, num_heads, num_kv_heads, head_size,
                            block_size, max_context_len, dtype);
  if (st != PA_OK) return st;
  if (!work_items || num_work_items < 1 ||
      num_work_items > static_cast<int64_t>(0x7fffffff) / num_kv_heads)
    return fail(PA_EINVAL, (std::string(who) + ": bad work list").c_str());
  if (!query_start_loc || !key || !value)
    return fail(PA_EINVAL, (std::string(who) + ": NULL query_start_loc, key or value").c_str());
  const int32_t eb = elem_bytes(dtype);
  const int64_t row = static_cast<int64_t>(num_kv_heads) * head_size;
  if (key_stride < row || value_stride < row || (key_stride * eb) % 16 != 0 ||
      (value_stride * eb) % 16 != 0 || !aligned16(key) || !aligned16(value))
    return fail(PA_EINVAL, (std::string(who) +
                            ": key/value rows must be 16-byte aligned with a stride of at "
                            "least num_kv_heads * head_size elements")
                               .c_str());
  pa::DecodeArgs a{out, query, key_cache, value_cache, block_tables, bt_stride, context_lens,
                   num_seqs, num_heads, num_kv_heads, head_size, block_size, 0, 1, scale, dtype,
                   nullptr, nullptr, nullptr, work_items, num_work_items};
  a.append = pa::dev::AppendArgs{query_start_loc, cow_src, static_cast<const uint4*>(key),
                                 static_cast<const uint4*>(value), key_stride * eb / 16,
                                 value_stride * eb / 16, static_cast<uint4*>(key_cache),
                                 static_cast<uint4*>(value_cache), slot_mapping};
  a.shared_blocks = shared_prefix_blocks;
  a.window = sliding_window;
  a.max_group = max_group;
  a.cascade_chunked = chunked;
  if (max_query_len > 0) {  // every new token is a query
    st = check_query_capacity(who, max_query_len, num_heads, num_kv_heads, head_size, dtype);
    if (st != PA_OK) return st;
    a.q_start = query_start_loc;
    a.max_query_len = max_query_len;
  } else if (max_query_len < 0) {
    return fail(PA_EINVAL, (std::string(who) + ": max_query_len must be >= 0").c_str());
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (partition_size == 0 && !chunked) return launched(pa::launch_decode(a, s), who);
  if (partition_size < 16 || partition_size > 4096 || partition_size % 16 != 0 ||
      partition_size % block_size != 0)
    return fail(PA_EINVAL, (std::string(who) + ": bad partition_size").c_str());
  // workspace rows: one per sequence, or num_seqs x max_query_len when every
  // new token is a query
  const int64_t out_rows = static_cast<int64_t>(num_seqs) * (max_query_len > 0 ? max_query_len : 1);
  if (out_rows > 0x7fffffff)
    return fail(PA_EINVAL, (std::string(who) + ": too many query rows").c_str());
  const size_t need = pa_split_workspace_bytes(static_cast<int32_t>(out_rows), num_heads,
                                               head_size, max_context_len, partition_size);
  if (!workspace || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(PA_EINVAL,
                (std::string(who) + ": workspace missing, too small or misaligned").c_str());
  set_split(a, workspace,
            split_layout(out_rows, num_heads, head_size, max_context_len, partition_size),
            partition_size);
  st = launched(pa::launch_decode(a, s), (std::string(who) + " (partition)").c_str());
  if (st != PA_OK) return st;
  return launched(pa::launch_split_reduce(a, s), (std::string(who) + " (reduce)").c_str());
}

int32_t pa_decode_step(void* out, const void* query, void* key_cache, void* value_cache,
                       const int32_t* block_tables, int64_t bt_stride,
                       const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                       int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                       int32_t max_context_len, float scale, int32_t dtype,
                       int32_t partition_size, const int32_t* work_items, int64_t num_work_items,
                       const int32_t* shared_prefix_blocks, void* workspace,
                       size_t workspace_bytes, const int32_t* query_start_loc,
                       const void* key, const void* value, int64_t key_stride,
                       int64_t value_stride, const int64_t* cow_src, int64_t* slot_mapping,
                       int32_t max_query_len, int32_t sliding_window, void* stream) {
  return decode_step_impl("pa_decode_step", 0, false, out, query, key_cache, value_cache,
                          block_tables,
                          bt_stride, context_lens, num_seqs, num_heads, num_kv_heads, head_size,
                          block_size, max_context_len, scale, dtype, partition_size, work_items,
                          num_work_items, shared_prefix_blocks, workspace, workspace_bytes,
                          query_start_loc, key, value, key_stride, value_stride, cow_src,
                          slot_mapping, max_query_len, sliding_window, stream);
}

static int32_t decode_step_cascade_impl(
    const char* who, bool chunked, void* out, const void* query, void* key_cache,
    void* value_cache, const int32_t* block_tables, int64_t bt_stride,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
    int32_t head_size, int32_t block_size, int32_t max_context_len, float scale, int32_t dtype,
    int32_t partition_size, const int32_t* plan, int64_t num_items, int32_t max_group_size,
    const int32_t* shared_prefix_blocks, void* workspace, size_t workspace_bytes,
    const int32_t* query_start_loc, const void* key, const void* value, int64_t key_stride,
    int64_t value_stride, const int64_t* cow_src, int64_t* slot_mapping, void* stream) {
  const std::string w(who);
  if (max_group_size < 0) return fail(PA_EINVAL, (w + ": max_group_size < 0").c_str());
  if ((dtype != PA_F16 && dtype != PA_BF16) || head_size != 128)
    return fail(PA_EINVAL,
                (w + ": group items need 16-bit storage and head_size 128").c_str());
  if (num_kv_heads < 1 || num_heads % num_kv_heads != 0 ||
      static_cast<int64_t>(max_group_size) * (num_heads / num_kv_heads) > 16)
    return fail(PA_EINVAL,
                (w + ": max_group_size x (num_heads / num_kv_heads) exceeds 16").c_str());
  if (chunked && partition_size == 0)
    return fail(PA_EINVAL, (w + ": a chunked plan needs its chunk_tokens as partition_size")
                               .c_str());
  return decode_step_impl(who, max_group_size, chunked, out, query, key_cache, value_cache,
                          block_tables, bt_stride, context_lens, num_seqs, num_heads,
                          num_kv_heads, head_size, block_size, max_context_len, scale, dtype,
                          partition_size, plan, num_items, shared_prefix_blocks, workspace,
                          workspace_bytes, query_start_loc, key, value, key_stride,
                          value_stride, cow_src, slot_mapping, 0, 0, stream);
}

int32_t pa_decode_step_cascade(void* out, const void* query, void* key_cache, void* value_cache,
                               const int32_t* block_tables, int64_t bt_stride,
                               const int32_t* context_lens, int32_t num_seqs,
                               int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                               int32_t block_size, int32_t max_context_len, float scale,
                               int32_t dtype, int32_t partition_size, const int32_t* plan,
                               int64_t num_items, int32_t max_group_size,
                               const int32_t* shared_prefix_blocks, void* workspace,
                               size_t workspace_bytes, const int32_t* query_start_loc,
                               const void* key, const void* value, int64_t key_stride,
                               int64_t value_stride, const int64_t* cow_src,
                               int64_t* slot_mapping, void* stream) {
  return decode_step_cascade_impl(
      "pa_decode_step_cascade", false, out, query, key_cache, value_cache, block_tables,
      bt_stride, context_lens, num_seqs, num_heads, num_kv_heads, head_size, block_size,
      max_context_len, scale, dtype, partition_size, plan, num_items, max_group_size,
      shared_prefix_blocks, workspace, workspace_bytes, query_start_loc, key, value, key_stride,
      value_stride, cow_src, slot_mapping, stream);
}

int32_t pa_decode_step_cascade_chunked(
    void* out, const void* query, void* key_cache, void* value_cache,
    const int32_t* block_tables, int64_t bt_stride, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
    int32_t block_size, int32_t max_context_len, float scale, int32_t dtype,
    int32_t chunk_tokens, const int32_t* plan, int64_t num_items, int32_t max_group_size,
    void* workspace, size_t workspace_bytes, const int32_t* query_start_loc, const void* key,
    const void* value, int64_t key_stride, int64_t value_stride, const int64_t* cow_src,
    int64_t* slot_mapping, void* stream) {
  return decode_step_cascade_impl(
      "pa_decode_step_cascade_chunked", true, out, query, key_cache, value_cache, block_tables,
      bt_stride, context_lens, num_seqs, num_heads, num_kv_heads, head_size, block_size,
      max_context_len, scale, dtype, chunk_tokens, plan, num_items, max_group_size, nullptr,
      workspace, workspace_bytes, query_start_loc, key, value, key_stride, value_stride, cow_src,
      slot_mapping, stream);
}

static int32_t attention_cascade_impl(const char* who, bool chunked, void* out,
                                      const void* query, const void* key_cache,
                                      const void* value_cache, const int32_t* block_tables,
                                      int64_t bt_stride, const int32_t* context_lens,
                                      int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                      int32_t head_size, int32_t block_size,
                                      int32_t max_context_len, float scale, int32_t dtype,
                                      int32_t partition_size, const int32_t* plan,
                                      int64_t num_items, int32_t max_group_size,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  const std::string w(who);
  int32_t st = check_decode(who, out, query, key_cache, value_cache, block_tables, bt_stride,
                            context_lens, num_seqs, num_heads, num_kv_heads, head_size,
                            block_size, max_context_len, dtype);
  if (st != PA_OK) return st;
  if (max_group_size < 0) return fail(PA_EINVAL, (w + ": max_group_size < 0").c_str());
  if ((dtype != PA_F16 && dtype != PA_BF16) || head_size != 128)
    return fail(PA_EINVAL,
                (w + ": group items need 16-bit storage and head_size 128").c_str());
  if (static_cast<int64_t>(max_group_size) * (num_heads / num_kv_heads) > 16)
    return fail(PA_EINVAL,
                (w + ": max_group_size x (num_heads / num_kv_heads) exceeds 16").c_str());
  if (!plan || num_items < 1 || num_items > static_cast<int64_t>(0x7fffffff) / num_kv_heads)
    return fail(PA_EINVAL, (w + ": bad plan").c_str());
  if (chunked && partition_size == 0)
    return fail(PA_EINVAL, (w + ": a chunked plan needs its chunk_tokens as partition_size")
                               .c_str());
  pa::DecodeArgs a{out, query, key_cache, value_cache, block_tables, bt_stride, context_lens,
                   num_seqs, num_heads, num_kv_heads, head_size, block_size, 0, 1, scale, dtype,
                   nullptr, nullptr, nullptr, plan, num_items};
  a.max_group = max_group_size;
  a.cascade_chunked = chunked;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (partition_size == 0) return launched(pa::launch_decode(a, s), who);
  if (partition_size < 16 || partition_size > 4096 || partition_size % 16 != 0 ||
      partition_size % block_size != 0)
    return fail(PA_EINVAL, (w + ": bad partition_size").c_str());
  const size_t need = pa_split_workspace_bytes(num_seqs, num_heads, head_size, max_context_len,
                                               partition_size);
  if (!workspace || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(PA_EINVAL, (w + ": workspace missing, too small or misaligned").c_str());
  set_split(a, workspace,
            split_layout(num_seqs, num_heads, head_size, max_context_len, partition_size),
            partition_size);
  st = launched(pa::launch_decode(a, s), (w + " (partition)").c_str());
  if (st != PA_OK) return st;
  return launched(pa::launch_split_reduce(a, s), (w + " (reduce)").c_str());
}

int32_t pa_paged_attention_cascade(void* out, const void* query, const void* key_cache,
                                   const void* value_cache, const int32_t* block_tables,
                                   int64_t bt_stride, const int32_t* context_lens,
                                   int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                   int32_t head_size, int32_t block_size,
                                   int32_t max_context_len, float scale, int32_t dtype,
                                   int32_t partition_size, const int32_t* plan,
                                   int64_t num_items, int32_t max_group_size, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  return attention_cascade_impl("pa_paged_attention_cascade", false, out, query, key_cache,
                                value_cache, block_tables, bt_stride, context_lens, num_seqs,
                                num_heads, num_kv_heads, head_size, block_size, max_context_len,
                                scale, dtype, partition_size, plan, num_items, max_group_size,
                                workspace, workspace_bytes, stream);
}

int32_t pa_paged_attention_cascade_chunked(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, int64_t bt_stride, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
    int32_t block_size, int32_t max_context_len, float scale, int32_t dtype,
    int32_t chunk_tokens, const int32_t* plan, int64_t num_items, int32_t max_group_size,
    void* workspace, size_t workspace_bytes, void* stream) {
  return attention_cascade_impl("pa_paged_attention_cascade_chunked", true, out, query,
                                key_cache, value_cache, block_tables, bt_stride, context_lens,
                                num_seqs, num_heads, num_kv_heads, head_size, block_size,
                                max_context_len, scale, dtype, chunk_tokens, plan, num_items,
                                max_group_size, workspace, workspace_bytes, stream);
}

int32_t pa_paged_attention_multi(void* out, const void* query, const void* key_cache,
                                 const void* value_cache, const int32_t* block_tables,
                                 int64_t bt_stride, const int32_t* context_lens,
                                 const int32_t* query_start_loc, int32_t num_seqs,
                                 int32_t max_query_len, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_size, int32_t block_size, int32_t max_context_len,
                                 float scale, int32_t dtype, int32_t partition_size,
                                 const int32_t* work_items, int64_t num_work_items,
                                 const int32_t* shared_prefix_blocks, void* workspace,
                                 size_t workspace_bytes, int64_t num_tokens,
                                 int32_t sliding_window, void* stream) {
  const char* who = "pa_paged_attention_multi";
  if (sliding_window < 0)
    return fail(PA_EINVAL, "pa_paged_attention_multi: sliding_window < 0");
  int32_t st = check_decode(who, out, query, key_cache, value_cache, block_tables, bt_stride,
                            context_lens, num_seqs, num_heads, num_kv_heads, head_size,
                            block_size, max_context_len, dtype);
  if (st != PA_OK) return st;
  if (!query_start_loc || num_tokens < 1)
    return fail(PA_EINVAL, "pa_paged_attention_multi: NULL query_start_loc or num_tokens < 1");
  st = check_query_capacity(who, max_query_len, num_heads, num_kv_heads, head_size, dtype);
  if (st != PA_OK) return st;
  if (!work_items || num_work_items < 1 ||
      num_work_items > static_cast<int64_t>(0x7fffffff) / num_kv_heads)
    return fail(PA_EINVAL, "pa_paged_attention_multi: bad work list");
  pa::DecodeArgs a{out, query, key_cache, value_cache, block_tables, bt_stride, context_lens,
                   num_seqs, num_heads, num_kv_heads, head_size, block_size, 0, 1, scale, dtype,
                   nullptr, nullptr, nullptr, work_items, num_work_items};
  a.shared_blocks = shared_prefix_blocks;
  a.q_start = query_start_loc;
  a.max_query_len = max_query_len;
  a.window = sliding_window;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (partition_size == 0) return launched(pa::launch_decode(a, s), who);
  if (partition_size < 16 || partition_size > 4096 || partition_size % 16 != 0 ||
      partition_size % block_size != 0)
    return fail(PA_EINVAL, "pa_paged_attention_multi: bad partition_size");
  if (num_tokens > 0x7fffffff) return fail(PA_EINVAL, "pa_paged_attention_multi: too many tokens");
  const size_t need = pa_split_workspace_bytes(static_cast<int32_t>(num_tokens), num_heads,
                                               head_size, max_context_len, partition_size);
  if (!workspace || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(PA_EINVAL, "pa_paged_attention_multi: workspace missing, too small or misaligned");
  set_split(a, workspace,
            split_layout(num_tokens, num_heads, head_size, max_context_len, partition_size),
            partition_size);
  st = launched(pa::launch_decode(a, s), "pa_paged_attention_multi (partition)");
  if (st != PA_OK) return st;
  return launched(pa::launch_split_reduce(a, s), "pa_paged_attention_multi (reduce)");
}

int32_t pa_paged_attention_partials(float* max_logits, float* exp_sums, float* partial_out,
                                    const void* query, const void* key_cache,
                                    const void* value_cache, const int32_t* block_tables,
                                    int64_t bt_stride, const int32_t* context_lens,
                                    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                    int32_t head_size, int32_t block_size,
                                    int32_t max_context_len, float scale, int32_t dtype,
                                    int32_t partition_size, const int32_t* work_items,
                                    int64_t num_work_items, const int32_t* shared_prefix_blocks,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  const char* who = "pa_paged_attention_partials";
  if (max_context_len < 0) return fail(PA_EINVAL, "pa_paged_attention_partials: bad sizes");
  const int32_t ctx = max_context_len > 0 ? max_context_len : 1;
  int32_t st = check_decode(who, partial_out, query, key_cache, value_cache, block_tables,
                            bt_stride, context_lens, num_seqs, num_heads, num_kv_heads,
                            head_size, block_size, ctx, dtype);
  if (st != PA_OK) return st;
  if (!max_logits || !exp_sums)
    return fail(PA_EINVAL, "pa_paged_attention_partials: NULL max_logits or exp_sums");
  if (partition_size < 16 || partition_size > 4096 || partition_size % 16 != 0 ||
      partition_size % block_size != 0)
    return fail(PA_EINVAL,
                "pa_paged_attention_partials: partition_size must be a multiple of 16 and of "
                "block_size, at most 4096");
  if (work_items && (num_work_items < 0 ||
                     num_work_items > static_cast<int64_t>(0x7fffffff) / num_kv_heads))
    return fail(PA_EINVAL, "pa_paged_attention_partials: bad work list");
  if (!work_items) {
    st = check_split_grid(who, num_seqs, num_kv_heads, ctx, partition_size);
    if (st != PA_OK) return st;
  }
  const int32_t np = (max_context_len + partition_size - 1) / partition_size;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  pa::DecodeArgs a{nullptr, query, key_cache, value_cache, block_tables, bt_stride,
                   context_lens, num_seqs, num_heads, num_kv_heads, head_size, block_size,
                   partition_size, np, scale, dtype, nullptr, nullptr, nullptr, work_items,
                   work_items ? num_work_items : 0};
  a.shared_blocks = shared_prefix_blocks;
  const bool any_work = np > 0 && (!work_items || num_work_items > 0);
  if (any_work) {
    const size_t need = pa_split_workspace_bytes(num_seqs, num_heads, head_size,
                                                 max_context_len, partition_size);
    if (!workspace || workspace_bytes < need ||
        reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
      return fail(PA_EINVAL,
                  "pa_paged_attention_partials: workspace missing, too small or misaligned");
    set_split(a, workspace,
              split_layout(num_seqs, num_heads, head_size, max_context_len, partition_size),
              partition_size);
    st = launched(pa::launch_decode(a, s), "pa_paged_attention_partials (partition)");
    if (st != PA_OK) return st;
  } else {
    // no key anywhere: the merge reads no part and writes (-inf, 0, 0)
    a.num_partitions = 0;
  }
  return launched(pa::launch_split_reduce_partials(a, max_logits, exp_sums, partial_out, s),
                  "pa_paged_attention_partials (merge)");
}

int32_t pa_merge_attention_partials(void* out, const float* max_logits, const float* exp_sums,
                                    const float* partial_out, int32_t num_parts,
                                    int32_t num_seqs, int32_t num_heads, int32_t head_size,
                                    int32_t dtype, void* stream) {
  const int32_t eb = elem_bytes(dtype);
  if (eb == 0) return fail(PA_EINVAL, "pa_merge_attention_partials: unknown dtype");
  if (!out || !max_logits || !exp_sums || !partial_out)
    return fail(PA_EINVAL, "pa_merge_attention_partials: NULL pointer");
  if (num_parts < 1 || num_seqs < 1 || num_heads < 1)
    return fail(PA_EINVAL, "pa_merge_attention_partials: bad sizes");
  if (static_cast<int64_t>(num_seqs) * ((num_heads + 3) / 4) > INT32_MAX)
    return fail(PA_EINVAL, "pa_merge_attention_partials: num_seqs x heads exceeds one launch's "
                           "workgroups");
  if (head_size != 64 && head_size != 128)
    return fail(PA_EINVAL, "pa_merge_attention_partials: head_size must be 64 or 128");
  if (reinterpret_cast<uintptr_t>(out) % eb != 0)
    return fail(PA_EINVAL, "pa_merge_attention_partials: out not aligned to its element size");
  if (reinterpret_cast<uintptr_t>(partial_out) % 8 != 0)
    return fail(PA_EINVAL, "pa_merge_attention_partials: partial_out not 8-byte aligned");
  return launched(pa::launch_merge_ranks(out, max_logits, exp_sums, partial_out, num_parts,
                                         num_seqs, num_heads, head_size, dtype,
                                         static_cast<hipStream_t>(stream)),
                  "pa_merge_attention_partials");
}

int32_t pa_prefill_block_tokens(int32_t num_heads, int32_t num_kv_heads, int32_t* tokens) {
  if (!tokens || num_heads < 1 || num_kv_heads < 1 || num_heads % num_kv_heads != 0)
    return fail(PA_EINVAL, "pa_prefill_block_tokens: bad arguments");
  const int32_t g = num_heads / num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8)
    return fail(PA_EINVAL, "pa_prefill_block_tokens: num_heads / num_kv_heads must be 1, 2, 4 or 8");
  *tokens = pa::prefill_block_tokens(g);
  return PA_OK;
}

// Shared checks of the prefill entry points; fills the launch arguments.
static int32_t check_prefill(const char* who, pa::PrefillArgs& a, int64_t bt_stride,
                             int32_t head_size, int32_t max_context_len) {
  const std::string w(who);
  if (a.window < 0) return fail(PA_EINVAL, (w + ": sliding_window < 0").c_str());
  int32_t st = check_decode(who, a.out, a.query, a.key_cache, a.value_cache, a.block_tables,
                            bt_stride, a.row_lens, a.num_rows, a.num_heads, a.num_kv_heads,
                            head_size, a.block_size, max_context_len, a.dtype);
  if (st != PA_OK) return st;
  if (!a.row_seq || !a.row_qsl) return fail(PA_EINVAL, (w + ": NULL row arrays").c_str());
  if (!(a.scale > 0.0f) || !std::isfinite(a.scale))
    return fail(PA_EINVAL, (w + ": scale must be positive and finite").c_str());
  if ((a.dtype != PA_F16 && a.dtype != PA_BF16) || head_size != 128)
    return fail(PA_EINVAL, (w + ": needs 16-bit storage and head_size 128").c_str());
  if (static_cast<int64_t>(a.num_rows) * a.num_kv_heads > 0x7fffffff)
    return fail(PA_EINVAL, (w + ": too many rows").c_str());
  return PA_OK;
}

int32_t pa_paged_attention_prefill(void* out, const void* query, const void* key_cache,
                                   const void* value_cache, const int32_t* block_tables,
                                   int64_t bt_stride, const int32_t* row_seq,
                                   const int32_t* row_lens, const int32_t* row_qsl,
                                   int32_t num_rows, int32_t num_heads, int32_t num_kv_heads,
                                   int32_t head_size, int32_t block_size,
                                   int32_t max_context_len, float scale, int32_t dtype,
                                   const int32_t* work_items, int32_t sliding_window,
                                   void* stream) {
  const char* who = "pa_paged_attention_prefill";
  pa::PrefillArgs a{out, query, key_cache, value_cache, block_tables, bt_stride, row_seq,
                    row_lens, row_qsl, work_items, num_rows, num_heads, num_kv_heads,
                    block_size, scale, dtype, sliding_window};
  const int32_t st = check_prefill(who, a, bt_stride, head_size, max_context_len);
  if (st != PA_OK) return st;
  return launched(pa::launch_prefill(a, static_cast<hipStream_t>(stream)), who);
}

int32_t pa_paged_attention_prefill_split(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, int64_t bt_stride, const int32_t* row_seq,
    const int32_t* row_lens, const int32_t* row_qsl, int32_t num_rows, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_size, int32_t block_size, int32_t max_context_len,
    float scale, int32_t dtype, const int32_t* work_items, int64_t num_work_items,
    int32_t partition_size, int32_t sliding_window, void* workspace, size_t workspace_bytes,
    int64_t num_tokens, void* stream) {
  const char* who = "pa_paged_attention_prefill_split";
  pa::PrefillArgs a{out, query, key_cache, value_cache, block_tables, bt_stride, row_seq,
                    row_lens, row_qsl, work_items, num_rows, num_heads, num_kv_heads,
                    block_size, scale, dtype, sliding_window};
  int32_t st = check_prefill(who, a, bt_stride, head_size, max_context_len);
  if (st != PA_OK) return st;
  if (!work_items || num_work_items < 1 ||
      num_work_items > static_cast<int64_t>(0x7fffffff) / num_kv_heads)
    return fail(PA_EINVAL, "pa_paged_attention_prefill_split: bad work list");
  if (partition_size < 16 || partition_size > 4096 || partition_size % 16 != 0 ||
      partition_size % block_size != 0)
    return fail(PA_EINVAL, "pa_paged_attention_prefill_split: bad partition_size");
  if (num_tokens < 1 || num_tokens > 0x7fffffff)
    return fail(PA_EINVAL, "pa_paged_attention_prefill_split: num_tokens out of range");
  const size_t need = pa_split_workspace_bytes(static_cast<int32_t>(num_tokens), num_heads,
                                               head_size, max_context_len, partition_size);
  if (!workspace || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(PA_EINVAL,
                "pa_paged_attention_prefill_split: workspace missing, too small or misaligned");
  const SplitLayout w =
      split_layout(num_tokens, num_heads, head_size, max_context_len, partition_size);
  // the merge: one output row per new token of each query-block row, over the
  // partitions below the row's length (from the row's window on)
  pa::DecodeArgs d{out, query, key_cache, value_cache, block_tables, bt_stride, row_lens,
                   num_rows, num_heads, num_kv_heads, head_size, block_size, 0, 1, scale, dtype,
                   nullptr, nullptr, nullptr, nullptr, 0};
  d.q_start = row_qsl;
  d.window = sliding_window;
  // a row holds up to 128 / G tokens: up to 32 merge workgroups per (row,
  // four heads), each taking every 32nd token
  d.merge_token_split = std::min(32, pa::prefill_block_tokens(num_heads / num_kv_heads));
  set_split(d, workspace, w, partition_size);
  a.partition_size = partition_size;
  a.num_partitions = w.np;
  a.num_items = num_work_items;
  a.ws_max = d.ws_max;
  a.ws_sum = d.ws_sum;
  a.ws_out = d.ws_out;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  st = launched(pa::launch_prefill(a, s), "pa_paged_attention_prefill_split (partitions)");
  if (st != PA_OK) return st;
  return launched(pa::launch_split_reduce(d, s), "pa_paged_attention_prefill_split (merge)");
}

int32_t pa_prefill_step(void* out, const void* query, void* key_cache, void* value_cache,
                        const int32_t* block_tables, int64_t bt_stride, const int32_t* row_seq,
                        const int32_t* row_lens, const int32_t* row_qsl, int32_t num_rows,
                        int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                        int32_t block_size, int32_t max_context_len, float scale, int32_t dtype,
                        const int32_t* work_items, int32_t sliding_window,
                        const int32_t* query_start_loc, const void* key, const void* value,
                        int64_t key_stride, int64_t value_stride, const int64_t* cow_src,
                        int64_t* slot_mapping, void* stream) {
  const char* who = "pa_prefill_step";
  pa::PrefillArgs a{out, query, key_cache, value_cache, block_tables, bt_stride, row_seq,
                    row_lens, row_qsl, work_items, num_rows, num_heads, num_kv_heads,
                    block_size, scale, dtype, sliding_window};
  int32_t st = check_prefill(who, a, bt_stride, head_size, max_context_len);
  if (st != PA_OK) return st;
  if (!query_start_loc || !key || !value)
    return fail(PA_EINVAL, "pa_prefill_step: NULL query_start_loc, key or value");
  const int32_t eb = elem_bytes(dtype);
  const int64_t row = static_cast<int64_t>(num_kv_heads) * head_size;
  if (key_stride < row || value_stride < row || (key_stride * eb) % 16 != 0 ||
      (value_stride * eb) % 16 != 0 || !aligned16(key) || !aligned16(value))
    return fail(PA_EINVAL, "pa_prefill_step: key/value rows must be 16-byte aligned with a "
                           "stride of at least num_kv_heads * head_size elements");
  if (key_stride * eb / 16 > INT32_MAX || value_stride * eb / 16 > INT32_MAX)
    return fail(PA_EINVAL, "pa_prefill_step: key/value row strides must stay below 2^35 bytes");
  a.append = pa::dev::AppendArgs{query_start_loc, cow_src, static_cast<const uint4*>(key),
                                 static_cast<const uint4*>(value), key_stride * eb / 16,
                                 value_stride * eb / 16, static_cast<uint4*>(key_cache),
                                 static_cast<uint4*>(value_cache), slot_mapping};
  return launched(pa::launch_prefill(a, static_cast<hipStream_t>(stream)), who);
}

int32_t pa_validate_tables(const int32_t* block_tables, int64_t bt_stride,
                           const int32_t* context_lens, int32_t num_seqs, int32_t block_size,
                           int32_t num_blocks, int32_t sliding_window, int32_t* result,
                           void* stream) {
  if (!block_tables || !context_lens || !result)
    return fail(PA_EINVAL, "pa_validate_tables: NULL pointer");
  if (num_seqs < 1 || bt_stride < 1 || block_size < 1 || num_blocks < 1 || sliding_window < 0)
    return fail(PA_EINVAL, "pa_validate_tables: bad sizes");
  return launched(pa::launch_validate_tables(block_tables, bt_stride, context_lens, num_seqs,
                                             block_size, num_blocks, sliding_window, result,
                                             static_cast<hipStream_t>(stream)),
                  "pa_validate_tables");
}

}  // extern "C"
