// Internal launchers of the HIP kernels, called by the ABI layer after it has
// validated every host-side argument.  Each returns hipSuccess or the launch
// error.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "decode_common.h"

namespace pa {

// cp_world = 1, cp_rank = 0, interleave = 1: the plain mapping.
hipError_t launch_slot_mapping(const int32_t* query_start_loc, const int64_t* positions,
                               const int32_t* block_tables, int64_t bt_stride, int32_t num_reqs,
                               int64_t num_tokens, int64_t max_num_tokens, int32_t block_size,
                               int32_t cp_world, int32_t cp_rank, int32_t interleave,
                               int64_t* slot_mapping, hipStream_t stream);

// elem_bytes: storage element size; row_elems = num_kv_heads * head_size.
hipError_t launch_reshape_and_cache(const void* key, const void* value, int64_t key_stride,
                                    int64_t value_stride, void* key_cache, void* value_cache,
                                    const int64_t* slot_mapping, int64_t num_tokens,
                                    int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                                    int32_t elem_bytes, hipStream_t stream);

hipError_t launch_copy_blocks(void* key_cache, void* value_cache, const int64_t* block_mapping,
                              int64_t num_pairs, int64_t block_bytes, hipStream_t stream);

// result: device int32 [2] = {invalid sequences, smallest invalid sequence or INT32_MAX}
hipError_t launch_validate_tables(const int32_t* block_tables, int64_t bt_stride,
                                  const int32_t* context_lens, int32_t num_seqs,
                                  int32_t block_size, int32_t num_blocks, int32_t window,
                                  int32_t* result, hipStream_t stream);

struct DecodeArgs {
  void* out;                 // final output (single pass) or nullptr
  const void* query;
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_tables;
  int64_t bt_stride;
  const int32_t* context_lens;
  int32_t num_seqs, num_heads, num_kv_heads, head_size, block_size;
  int32_t partition_size;    // tokens per partition (split) or 0 (single pass)
  int32_t num_partitions;    // NP (split) or 1
  float scale;
  int32_t dtype;
  float* ws_max;             // split workspace sections, or nullptr
  float* ws_sum;
  float* ws_out;
  const int32_t* items;      // work list [num_items][2] = (seq, partition), or nullptr
  int64_t num_items;
  dev::AppendArgs append{};  // the step's cache writes (append.qsl == nullptr: none)
  const int32_t* shared_blocks = nullptr;  // [S] leading blocks shared with other sequences
  const int32_t* q_start = nullptr;  // [S+1] new-token rows when every new token is a query
  int32_t max_query_len = 0;  // bound on q_start[s+1] - q_start[s] (host)
  int32_t window = 0;         // sliding window in tokens, 0 for none
  int32_t max_group = 0;      // members of the widest group item (cascade plan), 0 for none
  bool cascade_chunked = false;  // a chunked cascade plan on the single-pass kernel,
                                 // writing partials of partition_size-token slots
  int32_t merge_token_split = 1;  // workgroups per (row, head group) of the merge, each
                                  // merging every merge_token_split-th new token
};

// Query vectors one workgroup serves: (new tokens per sequence) x (query heads
// per KV head), rounded up to a power of two.
inline int query_vectors(const DecodeArgs& a) {
  const int per_seq = a.q_start ? (a.max_query_len > 0 ? a.max_query_len : 1) : 1;
  const int rows = a.max_group > per_seq ? a.max_group : per_seq;
  const int n = rows * (a.num_heads / a.num_kv_heads);
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

// Paged decode attention (single pass when partition_size == 0, else the
// partition kernel).  Picks the matrix-core kernel for grouped-query heads
// with 16-bit storage and head_size 128, the vector kernel otherwise; the
// choice can be forced where both apply (set_decode_kernel, or the
// environment variable PAGEDKV_DECODE_KERNEL=valu|mfma at start-up).
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
bool decode_mfma_supported(const DecodeArgs& a);
hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream);
// Single-pass cascade plan (items and group section as pa_decode_plan_cascade
// writes them with partition_size 0), or a chunked one
// (pa_decode_plan_cascade_chunked, cascade_chunked set: partials for the split
// merge): matrix cores, 16-bit storage, D = 128.
hipError_t launch_cascade_single(const DecodeArgs& a, hipStream_t stream);
// Prefill chunks on the matrix cores (16-bit storage, head_size 128): rows
// are query blocks of at most prefill_block_tokens(G) tokens (pa_query_blocks).
struct PrefillArgs {
  void* out;
  const void* query;
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_tables;
  int64_t bt_stride;
  const int32_t* row_seq;    // [num_rows] sequence of each row (its table row)
  const int32_t* row_lens;   // [num_rows] context length up to the row's last token
  const int32_t* row_qsl;    // [num_rows + 1] the rows' query rows
  const int32_t* work_items; // [num_rows][2] launch order (row, 0), or nullptr
  int32_t num_rows, num_heads, num_kv_heads, block_size;
  float scale;
  int32_t dtype;
  int32_t window;
  dev::AppendArgs append{};  // the step's cache writes (append.qsl == nullptr: none)
  // split launches (partition_size > 0): work_items holds num_items (row, p)
  // pairs and the partials go to the split workspace's three sections
  int32_t partition_size = 0, num_partitions = 0;
  int64_t num_items = 0;
  float* ws_max = nullptr;
  float* ws_sum = nullptr;
  float* ws_out = nullptr;
};
int prefill_block_tokens(int group);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
// mode: 0 automatic, 1 vector kernel, 2 matrix-core kernel; returns the previous mode.
int set_decode_kernel(int mode);
hipError_t launch_split_reduce(const DecodeArgs& a, hipStream_t stream);

// (m, l, o) of several parts per row (split partitions, or the ranks of a
// context-parallel group), with element strides between parts and rows.
struct PartView {
  const float* m;
  const float* l;
  const float* o;
  int64_t part_ml, row_ml;  // strides of m and l
  int64_t part_o, row_o;    // strides of o, in floats
};
// Destination of a merge: the storage-dtype output, or (out == nullptr) the
// merged (m, l, o) in fp32, rows [rows][H] and [rows][H][D].
struct MergeDst {
  void* out;
  float* m;
  float* l;
  float* o;
};

// The partitions of a split launch merged into one (m, l, o) per row instead
// of the final output.
hipError_t launch_split_reduce_partials(const DecodeArgs& a, float* m, float* l, float* o,
                                        hipStream_t stream);
// Rank-major parts ([num_parts][num_seqs][num_heads] and [..][head_size])
// merged into the storage-dtype output [num_seqs][num_heads][head_size].
hipError_t launch_merge_ranks(void* out, const float* m, const float* l, const float* o,
                              int32_t num_parts, int32_t num_seqs, int32_t num_heads,
                              int32_t head_size, int32_t dtype, hipStream_t stream);

}  // namespace pa
