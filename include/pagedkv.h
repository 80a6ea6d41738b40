/*
 * pagedkv.h — C ABI of the paged-KV decode library for MI355X (gfx950).
 *
 * The KV cache of every sequence lives in one pool of fixed-size physical
 * blocks of B token slots; a per-sequence block table maps logical block i to
 * an arbitrary physical block.  Sources (web pages on PagedAttention):
 *   [CSDN]      "PagedAttention 核心创新深度分析" (openeuler.csdn.net)
 *   [VLLBC]     "paged-attention-kv-cache" visual reading (blog.vllbc.top)
 *   [DEEPSONAR] "vLLM 的 PagedAttention：显存管理如何撑起大模型推理"
 *   [PUFANYI]   "Infra: PagedAttention" (pufanyi.com)
 *
 * Conventions shared by every call
 *   - Every call returns int32_t status: PA_OK, PA_EINVAL (a host-side
 *     argument is invalid: null pointer, unsupported size or dtype, bad
 *     alignment, unknown sequence), PA_ENOMEM (host allocator only: the pool
 *     is short; nothing was changed), PA_ELAUNCH (the HIP launch failed).
 *     Nothing aborts or throws across the ABI; pa_last_error() gives the
 *     message of the last failing call on the calling thread.
 *   - Device buffers are owned by the caller.  The library never allocates
 *     device memory; the split-K workspace is caller-provided.
 *   - Kernel launches are asynchronous on the caller's hipStream_t, passed as
 *     void* (NULL = the default stream).  A call returns once its kernels are
 *     enqueued.
 *   - Index data that lives on the device (block tables, slots, lengths,
 *     positions) is trusted: out-of-range values are undefined behaviour, as
 *     for any indirection a kernel follows.  Host-side sizes are validated.
 *   - KV cache layout (fixed by this ABI; the pages leave it open): key and
 *     value caches are each [num_blocks][num_kv_heads][B][head_size],
 *     row-major, elements of the storage dtype.  Slot s is row
 *     (s / B, :, s % B, :).  Both cache pointers must be 16-byte aligned.
 *   - Storage dtypes: PA_F32, PA_F16, PA_BF16.  Attention accumulates in fp32
 *     and rounds its output to the storage dtype (round to nearest even).
 *   - Query head h reads KV head h / (num_heads / num_kv_heads): groups of
 *     consecutive query heads share one KV head ([DEEPSONAR] section 2.1
 *     describes 64 query heads sharing 8 KV heads).
 *   - Supported shapes: head_size in {64, 128}; block_size in
 *     {1, 2, 4, 8, 16, 32, 64, 128}; num_heads / num_kv_heads in {1, 2, 4, 8}.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum pa_status { PA_OK = 0, PA_EINVAL = 1, PA_ENOMEM = 2, PA_ELAUNCH = 3 };
enum pa_dtype { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2 };

/* Library version string, e.g. "0.1.0". Static storage. */
const char* pa_version(void);
/* Name of a status code. Static storage. */
const char* pa_status_string(int32_t status);
/* Message of the last failing call on this thread ("" if none). Valid until
 * the next failing call on this thread. */
const char* pa_last_error(void);

/* ------------------------------------------------------------------------
 * Slot mapping.  [PUFANYI] "按 Block 分配": position p of a sequence is in
 * logical block p / B, found through the block table, at offset p % B.
 * [CSDN] section 2.3 (slot-mapping kernel, context-parallel world size 1):
 * slot = block_tables[r][p / B] * B + p % B for every scheduled token of
 * request r, the tokens of request r being [query_start_loc[r],
 * query_start_loc[r+1]).
 *
 *   query_start_loc  device int32 [num_reqs + 1], non-decreasing, from 0
 *   positions        device int64 [num_tokens], logical position per token
 *   block_tables     device int32 rows of bt_stride entries, one per request
 *   slot_mapping     device int64 [max_num_tokens] (output); entries
 *                    [num_tokens, max_num_tokens) are set to -1 (padding)
 *   num_tokens must equal query_start_loc[num_reqs].
 * One thread per slot_mapping entry finds its request by a binary search of
 * query_start_loc.
 * Errors: PA_EINVAL for null pointers, num_reqs < 1, num_tokens < 0,
 * max_num_tokens < num_tokens or > INT32_MAX, bt_stride < 1, block_size < 1.
 * ---------------------------------------------------------------------- */
int32_t pa_compute_slot_mapping(const int32_t* query_start_loc, const int64_t* positions,
                                const int32_t* block_tables, int64_t bt_stride,
                                int32_t num_reqs, int64_t num_tokens, int64_t max_num_tokens,
                                int32_t block_size, int64_t* slot_mapping, void* stream);

/* ------------------------------------------------------------------------
 * Context-parallel slot mapping.  [CSDN] section 2.3, the same kernel with a
 * context-parallel world of cp_world ranks: the ranks share one block table
 * whose entry j names a virtual block of B * cp_world positions
 * [j*B*cp_world, (j+1)*B*cp_world).  Offset o inside it is stored by rank
 * (o / interleave) % cp_world, in that rank's own cache, in the physical
 * block with the same number, at local offset
 * (o / (cp_world * interleave)) * interleave + o % interleave.  This call
 * gives rank cp_rank's slot for every scheduled token and -1 for the tokens
 * other ranks store, so pa_reshape_and_cache on the rank's cache writes only
 * its own tokens.  A rank's tokens fill its blocks in position order, so its
 * share of a sequence is an ordinary paged sequence over the same table,
 * pa_cp_local_context_lens tokens long.
 *
 *   Arguments as pa_compute_slot_mapping, plus
 *   cp_world     ranks, >= 1 (1 gives pa_compute_slot_mapping's result)
 *   cp_rank      this rank, 0 <= cp_rank < cp_world
 *   interleave   run length dealt to one rank at a time; must divide
 *                block_size (1: ranks alternate token by token; block_size:
 *                each rank takes B consecutive positions in turn)
 * Errors: as pa_compute_slot_mapping, plus PA_EINVAL for a bad cp_world,
 * cp_rank or interleave.
 * ---------------------------------------------------------------------- */
int32_t pa_compute_slot_mapping_cp(const int32_t* query_start_loc, const int64_t* positions,
                                   const int32_t* block_tables, int64_t bt_stride,
                                   int32_t num_reqs, int64_t num_tokens, int64_t max_num_tokens,
                                   int32_t block_size, int32_t cp_world, int32_t cp_rank,
                                   int32_t interleave, int64_t* slot_mapping, void* stream);

/* Host only: how many of the first context_lens[s] positions of each sequence
 * rank cp_rank stores under the mapping above (the rank-local context length
 * its attention call takes).  context_lens, local_lens: host int32
 * [num_seqs].  Errors: PA_EINVAL for null pointers, num_seqs < 0,
 * block_size < 1, a bad cp_world / cp_rank / interleave, a negative length. */
int32_t pa_cp_local_context_lens(const int32_t* context_lens, int32_t num_seqs,
                                 int32_t block_size, int32_t cp_world, int32_t cp_rank,
                                 int32_t interleave, int32_t* local_lens);

/* ------------------------------------------------------------------------
 * Cache scatter.  [VLLBC] walk-through of paper section 4.2 and [PUFANYI]
 * "按 Block 分配": each new token's key and value rows are stored at its
 * slot, filling the tail block.  Bit copy, no arithmetic.
 *
 *   key, value       device [num_tokens][key_stride] / [..][value_stride]
 *                    elements; token i's rows are [num_kv_heads][head_size]
 *                    contiguous starting at element i * stride
 *   slot_mapping     device int64 [num_tokens]; tokens with slot < 0 are
 *                    skipped; two tokens with the same slot race
 *   key_cache, value_cache  device caches (layout above), written in place
 * Errors: PA_EINVAL for null pointers, bad sizes or dtype, stride smaller
 * than num_kv_heads * head_size, misaligned caches.
 * ---------------------------------------------------------------------- */
int32_t pa_reshape_and_cache(const void* key, const void* value, int64_t key_stride,
                             int64_t value_stride, void* key_cache, void* value_cache,
                             const int64_t* slot_mapping, int64_t num_tokens,
                             int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                             int32_t dtype, void* stream);

/* ------------------------------------------------------------------------
 * Table check.  The kernels trust device-resident tables and lengths; this
 * call checks them on the device, for tests and debugging: a sequence is
 * invalid when its length is negative, when ceil(length / B) exceeds
 * bt_stride, or when a table entry the attention reads is outside
 * [0, num_blocks).  With sliding_window W > 0 the entries before the decode
 * query's window (positions below length - W) are not checked, since they
 * are never read and may be -1 (released); for several new tokens per
 * sequence pass W + max_query_len - 1.
 *   result  device int32 [2] (output): {number of invalid sequences, the
 *           smallest invalid sequence or INT32_MAX when none}; written by the
 *           call's own kernels (no prior initialisation needed)
 * Errors: PA_EINVAL for null pointers or sizes < 1 (sliding_window < 0).
 * ---------------------------------------------------------------------- */
int32_t pa_validate_tables(const int32_t* block_tables, int64_t bt_stride,
                           const int32_t* context_lens, int32_t num_seqs, int32_t block_size,
                           int32_t num_blocks, int32_t sliding_window, int32_t* result,
                           void* stream);

/* ------------------------------------------------------------------------
 * Block copy for copy-on-write.  [VLLBC] paper section 4.4 / Fig. 8 and
 * [PUFANYI] "共享前缀，分叉时 Copy-on-write": before a writer appends to a
 * shared, partly filled tail block, the whole physical block (all KV heads,
 * all B slots, key and value) is copied into a fresh block.
 *
 *   block_mapping    device int64 [num_pairs][2] = (src, dst) block ids; a
 *                    dst must not repeat nor be another pair's src
 * Errors: PA_EINVAL for null pointers, num_pairs < 0, bad sizes or dtype.
 * num_pairs == 0 launches nothing.
 * ---------------------------------------------------------------------- */
int32_t pa_copy_blocks(void* key_cache, void* value_cache, const int64_t* block_mapping,
                       int64_t num_pairs, int32_t num_kv_heads, int32_t head_size,
                       int32_t block_size, int32_t dtype, void* stream);

/* ------------------------------------------------------------------------
 * Paged decode attention, single pass.  [VLLBC] walk-through of paper
 * sections 4.1-4.2: the new query token of every sequence is scored against
 * all of its cached keys, read block by block through the block table; the
 * scores go through a softmax and weight the cached values.  [PUFANYI]
 * closing section: the result is that of dense attention over the same
 * tokens.  Per (sequence s, query head h), with g = h / (H / H_kv):
 *   x_t = scale * <query[s][h], K[s][g][t]>,  t < context_lens[s]
 *   out[s][h] = sum_t softmax(x)_t * V[s][g][t]
 *
 *   out, query       device [num_seqs][num_heads][head_size], storage dtype
 *   block_tables     device int32 rows of bt_stride entries; row s needs
 *                    ceil(context_lens[s] / B) valid block ids
 *   context_lens     device int32 [num_seqs], each in [1, max_context_len]
 *   max_context_len  host bound on context_lens (used to size launches)
 * Errors: PA_EINVAL for null pointers, unsupported shapes or dtype,
 * num_heads % num_kv_heads != 0, max_context_len < 1, or more workgroups
 * than one launch holds (num_seqs x num_kv_heads, or num_seqs x
 * ceil(num_heads / 4) for a merge, above INT32_MAX); every attention call
 * shares these checks.
 * ---------------------------------------------------------------------- */
int32_t pa_paged_attention_decode(void* out, const void* query, const void* key_cache,
                                  const void* value_cache, const int32_t* block_tables,
                                  int64_t bt_stride, const int32_t* context_lens,
                                  int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                  int32_t head_size, int32_t block_size,
                                  int32_t max_context_len, float scale, int32_t dtype,
                                  void* stream);

/* Kernel choice for the attention calls (process-wide, not thread-safe):
 * 0 = automatic (matrix-core kernel for grouped-query heads, num_heads /
 * num_kv_heads >= 2, with 16-bit storage and head_size 128; vector kernel
 * otherwise), 1 = vector kernel always, 2 = matrix-core kernel wherever it
 * applies (16-bit storage, head_size 128).  Every choice computes the same
 * result within the stated tolerances.  The initial mode comes from the
 * environment variable PAGEDKV_DECODE_KERNEL=valu|mfma if set, else 0.
 * Returns the previous mode, or -1 (mode unchanged) for a mode outside 0..2. */
int32_t pa_set_decode_kernel(int32_t mode);

/* ------------------------------------------------------------------------
 * Split-K variant for long contexts.  The pages do not describe it; it is
 * the standard partition/merge of a softmax: the context of each sequence is
 * cut at logical positions into partitions of partition_size tokens; a first
 * kernel computes per (s, h, partition p) m_p = max x, l_p = sum exp(x - m_p)
 * and o_p = sum exp(x - m_p) v / l_p over the partition; a second kernel
 * merges them with M = max m_p, a_p = l_p exp(m_p - M),
 * out = sum a_p o_p / sum a_p.  Same result as the single pass up to
 * rounding.
 *
 * pa_split_workspace_bytes gives the workspace size for a launch (host call).
 * Workspace contents (fp32, caller-owned, no initialisation needed):
 *   max_logits [num_seqs][num_heads][NP], exp_sums [num_seqs][num_heads][NP],
 *   tmp_out [num_seqs][num_heads][NP][head_size],
 *   NP = ceil(max_context_len / partition_size), sections 256-byte aligned.
 * partition_size must be a multiple of block_size and of 16, at most 4096.
 * Errors: as pa_paged_attention_decode, plus PA_EINVAL for a bad
 * partition_size, a null workspace or workspace_bytes too small.
 * ---------------------------------------------------------------------- */
size_t pa_split_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_size,
                                int32_t max_context_len, int32_t partition_size);
/* Host: where the three sections of that workspace start, for a caller that
 * reads the partials.  offsets_out (host int64 [3]) receives the byte offsets
 * of max_logits, exp_sums and tmp_out; *num_partitions_out receives NP.
 * num_seqs counts the workspace's rows (sequences, or new tokens when every
 * new token is a query).  PA_EINVAL for null outputs or sizes < 1. */
int32_t pa_split_workspace_layout(int32_t num_seqs, int32_t num_heads, int32_t head_size,
                                  int32_t max_context_len, int32_t partition_size,
                                  int64_t* offsets_out, int32_t* num_partitions_out);

int32_t pa_paged_attention_decode_split(void* out, const void* query, const void* key_cache,
                                        const void* value_cache, const int32_t* block_tables,
                                        int64_t bt_stride, const int32_t* context_lens,
                                        int32_t num_seqs, int32_t num_heads,
                                        int32_t num_kv_heads, int32_t head_size,
                                        int32_t block_size, int32_t max_context_len,
                                        float scale, int32_t dtype, int32_t partition_size,
                                        void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * pa_paged_attention_decode_split without the workspace arguments.  The
 * split workspace is a static device array of PA_NOALLOC_WORKSPACE_BYTES
 * inside the library (each GPU the library runs on holds one until the
 * process ends); the call allocates nothing and calls no allocating routine.
 * The caller still passes inputs and outputs, as for
 * pa_paged_attention_decode_split, and gets the same result bit for bit.
 * The array keeps the last call's partials; nothing needs clearing (every
 * partition a merge reads is written first).  Calls that overlap on one GPU
 * (two streams, or two threads) share the array and race: serialise them.
 * Errors: as pa_paged_attention_decode_split, plus PA_EINVAL when
 * pa_split_workspace_bytes(num_seqs, num_heads, head_size, max_context_len,
 * partition_size) exceeds PA_NOALLOC_WORKSPACE_BYTES (checked before any
 * device call) or the current device index is 64 or more; PA_ELAUNCH when
 * the array's device address cannot be found on the current device.
 * ---------------------------------------------------------------------- */
#define PA_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)
int32_t pa_paged_attention_decode_split_noalloc(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, int64_t bt_stride, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
    int32_t block_size, int32_t max_context_len, float scale, int32_t dtype,
    int32_t partition_size, void* stream);

/* ------------------------------------------------------------------------
 * Planned launch (load balance).  The two calls above launch one workgroup
 * per (sequence, KV head[, partition]) in index order, including partitions
 * past a sequence's end.  With lengths that vary a lot, a launch that starts
 * the largest pieces of work first and contains no empty pieces finishes
 * sooner; this pair of calls provides that.  Same results as the calls above.
 *
 * pa_decode_plan (host only): from host context lengths, the list of every
 * non-empty (sequence, partition) item — one item (s, 0) per sequence when
 * partition_size == 0 — ordered by decreasing token count, counted in
 * buckets of 256 tokens; items of one bucket keep (sequence, partition)
 * order so that neighbouring sequences, e.g. forks sharing a prompt, stay
 * together.  items: host int32 [capacity][2]; *num_items receives the
 * item count.  items == NULL only queries the count.  PA_EINVAL for a null
 * context_lens/num_items, num_seqs < 1, a negative length, a length of 0
 * with partition_size == 0, partition_size < 0, or a capacity below the
 * count.  With partition_size > 0 a sequence of length 0 (an empty
 * rank-local share under context parallelism) has no item; the split
 * attention output of such a sequence is 0.
 *
 * pa_paged_attention_decode_planned: attention driven by such a list (copied
 * to the device by the caller: work_items = device int32 [num_work_items][2]).
 * partition_size == 0: single pass, the list must name every sequence once
 * as (s, 0) and workspace may be NULL.  partition_size > 0: the split-K
 * kernels (same rules and workspace as pa_paged_attention_decode_split); the
 * list must name every non-empty partition once.  Items missing from the
 * list leave their outputs undefined (no out-of-bounds access).
 * shared_prefix_blocks (device int32 [num_seqs], may be NULL): how many
 * leading blocks of each sequence's table other sequences also read (forks
 * of one prompt, [VLLBC] paper section 4.4).  K/V rows of those blocks are
 * loaded through the caches so that the sharers reuse them; all other rows
 * are read once and are loaded as non-temporal streams.  A cache hint only:
 * results do not depend on it.  NULL = nothing shared.  The unplanned calls
 * above stream every row.
 *
 * Sliding window ([CSDN] sections 3.1.1 and 3.3.1 release the blocks a
 * sliding window leaves behind; the rule itself is this library's reading):
 * sliding_window W > 0 makes a query at position p attend only to positions
 * p - W + 1 .. p, the W most recent tokens with itself; 0 is full attention.
 * Only the K/V rows inside the window are read, so table entries before it
 * may be -1 (blocks released by pa_pool_remove_skipped).  With
 * partition_size > 0 the partitions wholly before the window have no item
 * and are not launched or merged.
 *
 * pa_decode_plan_window: pa_decode_plan for windowed attention and grouped
 * readers.  query_lens (host int32 [num_seqs], NULL = one query per
 * sequence) gives each sequence's new-token count n_s, 1 <= n_s <= its
 * length; its first query (position L_s - n_s) starts the window.  An
 * item's size is the part of it inside the window.  group_keys (host int32
 * [num_seqs], may be NULL = the sequence index) order the items of one size
 * bucket by key, then by (sequence, partition): sequences that read one
 * shared prefix (e.g. key = the prefix's first block) then run together
 * wherever they sit in the batch.  sliding_window == 0 and NULL query_lens
 * and group_keys give pa_decode_plan's list.
 * ---------------------------------------------------------------------- */
int32_t pa_decode_plan(const int32_t* context_lens, int32_t num_seqs, int32_t partition_size,
                       int32_t* items, int64_t capacity, int64_t* num_items);

int32_t pa_decode_plan_window(const int32_t* context_lens, const int32_t* query_lens,
                              const int32_t* group_keys, int32_t num_seqs,
                              int32_t partition_size, int32_t sliding_window, int32_t* items,
                              int64_t capacity, int64_t* num_items);

/* ------------------------------------------------------------------------
 * Cascade plan (host): a decode batch in which several sequences read one
 * prefix of physical blocks (the samples of one prompt, [VLLBC] paper
 * section 4.4; requests that share cached prefix blocks) computes the
 * partitions lying wholly inside that prefix once per group of sharers
 * instead of once per sequence.  The result is the same attention: a
 * sequence's partitions are merged exactly as in the split launch, whether a
 * group item or its own item wrote them.
 *   context_lens   host int32 [num_seqs], lengths after the step
 *   block_tables   host int32 [num_seqs][bt_stride], the step's tables
 *   new_tokens     host int32 [num_seqs] (NULL = 1 each): rows written during
 *                  the step, the last new_tokens[s] positions of sequence s
 * Sequences whose first table entry is the same block form a candidate
 * group.  Its prefix is the run of leading entries every member has, cut to
 * full blocks that end before any member's first new token; the group is
 * split into chunks of at most max_group_size members.  With partition_size
 * > 0 (a multiple of block_size) the partitions wholly inside the prefix
 * become group items (-1 - c, partition) of chunk c, and every other
 * (sequence, partition) pair keeps its own item.  With partition_size == 0
 * (single pass) chunk c has the one item (-1 - c, prefix tokens), which
 * reads the prefix once and then each member's own tokens, and every
 * sequence outside a chunk has the item (s, 0).  Output `plan` (host int32,
 * capacity entries), plan_len entries in all:
 *   [2 * num_items]  items, largest first: with partitions as in
 *                    pa_decode_plan (by the tokens they read, in buckets of
 *                    256); single pass by the tokens they read counted in
 *                    16-token tiles per piece (no buckets), ties in batch
 *                    order of their first sequence
 *   [1]              number of chunks C
 *   [C + 1]          offsets of the chunks' member lists
 *   [offsets[C]]     members (batch rows)
 * max_members receives the widest chunk (0 when no group formed; the plan is
 * then an ordinary item list followed by an empty group section).  plan ==
 * NULL returns only num_items, plan_len and max_members.
 * Errors: PA_EINVAL for null outputs, sizes < 1, a partition_size < 0 or not
 * a multiple of block_size, new tokens outside [1, length], a table row
 * shorter than its length, or capacity < plan_len.
 * ---------------------------------------------------------------------- */
int32_t pa_decode_plan_cascade(const int32_t* context_lens, const int32_t* block_tables,
                               int64_t bt_stride, const int32_t* new_tokens, int32_t num_seqs,
                               int32_t block_size, int32_t partition_size,
                               int32_t max_group_size, int32_t* plan, int64_t capacity,
                               int64_t* num_items, int64_t* plan_len, int32_t* max_members);
/* Host: the widest max_group_size the cascade calls take for this shape,
 * members x (num_heads / num_kv_heads) <= 16 (the matrix cores' columns of a
 * group item), at most 8; 0 for fp32 storage or a head_size other than 128,
 * which have no group-item kernels.  *group receives it.  PA_EINVAL for a
 * null group or bad head counts. */
int32_t pa_cascade_max_group(int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                             int32_t dtype, int32_t* group);

int32_t pa_paged_attention_decode_planned(void* out, const void* query, const void* key_cache,
                                          const void* value_cache, const int32_t* block_tables,
                                          int64_t bt_stride, const int32_t* context_lens,
                                          int32_t num_seqs, int32_t num_heads,
                                          int32_t num_kv_heads, int32_t head_size,
                                          int32_t block_size, int32_t max_context_len,
                                          float scale, int32_t dtype, int32_t partition_size,
                                          const int32_t* work_items, int64_t num_work_items,
                                          const int32_t* shared_prefix_blocks, void* workspace,
                                          size_t workspace_bytes, int32_t sliding_window,
                                          void* stream);

/* ------------------------------------------------------------------------
 * One decode step in one launch (plus the reduce when partition_size > 0).
 * Does what pa_copy_blocks, pa_compute_slot_mapping, pa_reshape_and_cache and
 * pa_paged_attention_decode_planned do in sequence, for the usual decode
 * shape of the step: sequence s appends n_s = query_start_loc[s+1] -
 * query_start_loc[s] tokens at positions [L_s - n_s, L_s), L_s =
 * context_lens[s] (lengths after the step), their K/V rows being rows
 * query_start_loc[s] .. of key / value; when cow_src[s] >= 0, the block of
 * position L_s - n_s (a fresh copy-on-write block, [VLLBC] paper section
 * 4.4 / Fig. 8) first receives the slots before that position from block
 * cow_src[s].  Each attention workgroup writes the rows it then reads, so
 * slot_mapping, out and every cache slot below L_s end exactly as with the
 * four separate calls.  The slots at or past L_s of a copied block, which
 * pa_copy_blocks fills from the source block, are left unspecified here
 * (no step reads a slot before writing it).
 *   key_cache, value_cache  written in place
 *   query_start_loc  device int32 [num_seqs + 1]
 *   key, value       device, 16-byte aligned rows [T][num_kv_heads][head_size]
 *                    with token strides key_stride / value_stride (elements,
 *                    a multiple of 16 bytes)
 *   cow_src          device int64 [num_seqs], -1 for none; may be NULL
 *   slot_mapping     device int64 [T] receiving the new tokens' slots; may be NULL
 *   max_query_len    0: one query per sequence (query / out [num_seqs][H][D],
 *                    the decode case); > 0: every new token is a query with
 *                    the causal rule of pa_paged_attention_multi (query / out
 *                    [T][H][D], at most max_query_len new tokens per
 *                    sequence; split-K workspace sized for num_seqs x
 *                    max_query_len rows)
 * The other arguments are those of pa_paged_attention_decode_planned
 * (sliding_window included: the copy-on-write rows and new tokens are written
 * whatever the window, since they lie in the partition of the first new
 * token, which is always inside it).
 * ---------------------------------------------------------------------- */
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
                       int32_t max_query_len, int32_t sliding_window, void* stream);

/* ------------------------------------------------------------------------
 * pa_decode_step over a cascade plan (pa_decode_plan_cascade): one query per
 * sequence, no sliding window, partition_size the plan's.  A group item
 * reads each K/V tile of its shared prefix once for all its members (their
 * queries are the columns of the matrix-core tiles).  Split plans
 * (partition_size > 0): it writes every member's partial to that member's
 * workspace slot, merged as in the split launch.  Single-pass plans
 * (partition_size == 0, workspace may be NULL): it goes on with each
 * member's own tokens and writes every member's output; it also writes the
 * new rows of all its members first, which serializes those writes on a few
 * workgroups (pa_paged_attention_cascade after pa_copy_blocks and
 * pa_reshape_and_cache spreads them over the whole GPU).  The rest is
 * pa_decode_step.
 *   plan            device int32, the whole cascade plan (items and group
 *                   section), unchanged during the call
 *   num_items       its item count
 *   max_group_size  its max_members (0: no group item)
 * Needs 16-bit storage, head_size 128 and max_group_size x (num_heads /
 * num_kv_heads) <= 16.  Errors: those of pa_decode_step, plus PA_EINVAL for
 * another dtype or head size, or a group too wide.
 * ---------------------------------------------------------------------- */
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
                               int64_t* slot_mapping, void* stream);

/* ------------------------------------------------------------------------
 * Chunked cascade plans: the single-pass cascade's workgroup per (group, KV
 * head) reads a whole shared prefix, so a batch of few groups is one round
 * of long workgroups.  A chunked plan cuts each group's prefix into pieces of
 * chunk_tokens (a multiple of block_size and of 16, at most 4096), each read
 * once for all members by a workgroup of its own, and gives the group one
 * more item that reads the rest of the prefix once and then every member's
 * own tokens (the step's writes happen there, as in the single-pass
 * cascade).  Every item writes (m, l, o) partials; the split merge over
 * ceil(L / chunk_tokens) parts per sequence gives the same attention
 * ([VLLBC] paper section 4.4 / Fig. 8: the samples of one prompt share its
 * blocks; the result is the plain attention of each sequence).
 *
 * pa_decode_plan_cascade_chunked (host): groups as pa_decode_plan_cascade
 * forms them.  Items, largest first:
 *   (-1 - c, j), j < pf_c = prefix_c / chunk_tokens: chunk c's prefix tokens
 *        [j * chunk_tokens, (j + 1) * chunk_tokens), written to slot j
 *   (-1 - c, pf_c): tokens [pf_c * chunk_tokens, prefix_c) for all members,
 *        then each member's [prefix_c, L_m), written to slot pf_c (the
 *        member's later slots are marked empty)
 *   (s, p) for a sequence outside every chunk: tokens [p * chunk_tokens,
 *        min((p + 1) * chunk_tokens, L_s)), written to slot p
 * Layout of plan: [2 * num_items] items, [1] C, [C + 1] member offsets, [C]
 * prefix tokens of each chunk, members.  Arguments and errors as
 * pa_decode_plan_cascade, with chunk_tokens >= 1 in place of partition_size.
 *
 * pa_decode_step_cascade_chunked: pa_decode_step_cascade over such a plan,
 * chunk_tokens in place of partition_size, workspace as for
 * pa_paged_attention_decode_split with partition_size = chunk_tokens; the
 * cascade launch plus the merge launch.  pa_paged_attention_cascade_chunked:
 * the attention alone (caches already written).  Errors as their unchunked
 * counterparts, plus PA_EINVAL for chunk_tokens == 0.
 * ---------------------------------------------------------------------- */
/* pa_cascade_auto_chunk (host): the chunk_tokens a step would take on its
 * own: 2048 when the single-pass plan gives fewer than 512 (item, KV head)
 * workgroups (one round at two per compute unit) and some group's prefix
 * spans at least 4096 tokens, else 0 (the single-pass plan).  Arguments as
 * pa_decode_plan_cascade, plus num_kv_heads; *chunk_tokens receives it. */
int32_t pa_cascade_auto_chunk(const int32_t* context_lens, const int32_t* block_tables,
                              int64_t bt_stride, const int32_t* new_tokens, int32_t num_seqs,
                              int32_t block_size, int32_t max_group_size, int32_t num_kv_heads,
                              int32_t* chunk_tokens);
int32_t pa_decode_plan_cascade_chunked(const int32_t* context_lens, const int32_t* block_tables,
                                       int64_t bt_stride, const int32_t* new_tokens,
                                       int32_t num_seqs, int32_t block_size,
                                       int32_t chunk_tokens, int32_t max_group_size,
                                       int32_t* plan, int64_t capacity, int64_t* num_items,
                                       int64_t* plan_len, int32_t* max_members);
int32_t pa_decode_step_cascade_chunked(
    void* out, const void* query, void* key_cache, void* value_cache,
    const int32_t* block_tables, int64_t bt_stride, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
    int32_t block_size, int32_t max_context_len, float scale, int32_t dtype,
    int32_t chunk_tokens, const int32_t* plan, int64_t num_items, int32_t max_group_size,
    void* workspace, size_t workspace_bytes, const int32_t* query_start_loc, const void* key,
    const void* value, int64_t key_stride, int64_t value_stride, const int64_t* cow_src,
    int64_t* slot_mapping, void* stream);
int32_t pa_paged_attention_cascade_chunked(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, int64_t bt_stride, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
    int32_t block_size, int32_t max_context_len, float scale, int32_t dtype,
    int32_t chunk_tokens, const int32_t* plan, int64_t num_items, int32_t max_group_size,
    void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Query blocks (host) for steps whose sequences bring more new tokens than
 * one workgroup holds as query vectors (max_query_len x (num_heads /
 * num_kv_heads) above 16, or 8 for the vector kernel): a prefill chunk
 * ([DEEPSONAR] section 2.5 schedules prefill chunks like decode tokens;
 * [CSDN] section 2.3 lays a step's tokens out by query_start_loc).  Sequence
 * s's n_s new tokens are cut into blocks of at most max_block tokens; block j
 * is a row of its own for pa_paged_attention_multi, over sequence s's table
 * row, with the new tokens rows [query_start_loc[s] + j*max_block, ...) and
 * the context length L_s - n_s + (end of the block), so every token keeps its
 * causal bound.  Output rows keep the step's token order.  Blocks of one
 * sequence read each other's new rows, so the cache writes of such a step go
 * first (pa_reshape_and_cache), not inside the attention launch.
 *   context_lens, query_start_loc  host int32 [num_seqs], [num_seqs + 1]
 *   row_seq, row_lens              host int32 [capacity] (outputs): source
 *                                  sequence and context length of each row
 *   row_qsl                        host int32 [capacity + 1] (output)
 * row_seq == NULL returns only num_rows.  Errors: PA_EINVAL for null
 * arguments, num_seqs or max_block < 1, new tokens outside [1, length],
 * capacity < num_rows.
 * ---------------------------------------------------------------------- */
int32_t pa_query_blocks(const int32_t* context_lens, const int32_t* query_start_loc,
                        int32_t num_seqs, int32_t max_block, int32_t* row_seq,
                        int32_t* row_lens, int32_t* row_qsl, int64_t capacity,
                        int64_t* num_rows);
/* pa_query_block_hints (host): the shared-block cache hint
 * (shared_prefix_blocks of pa_paged_attention_multi) of query-block rows.
 * The rows of a sequence cut into several blocks all read every block of its
 * context, so such a row's hint covers its whole context,
 * ceil(row_lens[r] / block_size) blocks; a sequence left in one row keeps
 * its own hint seq_shared_blocks[row_seq[r]] (NULL: 0).
 *   row_seq, row_lens   host int32 [num_rows], as pa_query_blocks wrote them
 *   seq_shared_blocks   host int32 [num_seqs] or NULL
 *   row_shared_out      host int32 [num_rows] (output)
 * PA_EINVAL for null arrays, sizes < 1, or a row whose sequence is outside
 * [0, num_seqs) or whose length is negative. */
int32_t pa_query_block_hints(const int32_t* row_seq, const int32_t* row_lens, int32_t num_rows,
                             const int32_t* seq_shared_blocks, int32_t num_seqs,
                             int32_t block_size, int32_t* row_shared_out);

/* pa_prefill_plan (host): the launch order of pa_paged_attention_prefill and
 * pa_prefill_step over query-block rows, as their work_items list.  A row's
 * size is the number of keys it reads (its length, or with a sliding window
 * W the positions from its first query's window on); the rows of a sequence
 * go together, sequences by their largest row, largest first (ties by
 * sequence index), and within a sequence largest row first.  The rows of a
 * sequence read the same K/V rows, so launched together they find them in
 * the caches, and large pieces of work first leave small ones to fill the
 * end of the launch.  Each workgroup computes one (row, KV head) whatever
 * the order: results do not depend on it.
 *   row_seq, row_lens   host int32 [num_rows], as pa_query_blocks wrote them
 *   row_qlens           host int32 [num_rows]: new tokens of each row
 *                       (row_qsl[r + 1] - row_qsl[r]), or NULL = 1
 *   sliding_window      as for pa_paged_attention_prefill (0 = none)
 *   items               host int32 [num_rows][2] (output): (row, 0) pairs
 * PA_EINVAL for null arrays, num_rows < 1, sliding_window < 0, a negative
 * sequence index or length, or a row whose new tokens are outside
 * [0, length]. */
int32_t pa_prefill_plan(const int32_t* row_seq, const int32_t* row_lens,
                        const int32_t* row_qlens, int32_t num_rows, int32_t sliding_window,
                        int32_t* items);

/* pa_prefill_plan_split (host): the work list of pa_paged_attention_prefill_split,
 * (row, p) pairs: for each row the partitions of partition_size keys from
 * the one holding its first visible key (0, or with a sliding window W the
 * start of its first query's window) to the one holding its last key
 * (ceil(row_lens[r] / partition_size) - 1).  The rows of a sequence go
 * together, sequences by their largest row (keys read), largest first, and
 * within a sequence by partition, then by row size.
 *   row_seq, row_lens, row_qlens, sliding_window   as for pa_prefill_plan
 *   items        host int32 [capacity][2] (output), or NULL to count only
 *   num_items    host (output): the number of items
 * PA_EINVAL for null row arrays or num_items, num_rows < 1,
 * sliding_window < 0, partition_size < 1, a negative sequence index, a
 * length below 1, new tokens outside [0, length], or a capacity below the
 * count. */
int32_t pa_prefill_plan_split(const int32_t* row_seq, const int32_t* row_lens,
                              const int32_t* row_qlens, int32_t num_rows, int32_t sliding_window,
                              int32_t partition_size, int32_t* items, int64_t capacity,
                              int64_t* num_items);

/* pa_prefill_auto_partition (host): the partition size a caller without one
 * should give the split prefill, or 0 for one pass.  4096 when the rows
 * would give fewer (row, KV head) workgroups than two per CU of an MI355X
 * (512) and the longest row holds at least 8192 keys (and 4096 is a
 * multiple of block_size), else 0.  (One sequence of 32k keys taking a
 * 512-token chunk: 128 workgroups on a 32-KV-head layer; its split launch is
 * 2.3x faster than the one pass.)  PA_EINVAL for a null output,
 * num_rows, num_kv_heads or block_size below 1, or a negative length. */
int32_t pa_prefill_auto_partition(int32_t num_rows, int32_t num_kv_heads, int32_t max_row_len,
                                  int32_t block_size, int32_t* partition_size);

/* ------------------------------------------------------------------------
 * Prefill attention over query blocks on the matrix cores (16-bit storage,
 * head_size 128, single pass): the result of pa_paged_attention_multi for
 * the rows of pa_query_blocks, computed with each key/value tile loaded once
 * into LDS for all query vectors of a block instead of once per 16 of them.
 *
 * pa_prefill_block_tokens (host): *tokens receives the max_block to give
 * pa_query_blocks, 128 / (num_heads / num_kv_heads) new tokens per block.
 * PA_EINVAL for a null tokens or a head ratio other than 1, 2, 4 or 8.
 *
 * pa_paged_attention_prefill: one workgroup per (row, KV head).
 *   out, query          device [num_tokens][num_heads][128], the step's tokens
 *   block_tables        device int32 [num_seqs][bt_stride], indexed by row_seq
 *   row_seq, row_lens   device int32 [num_rows]: each row's table row and its
 *                       context length (that of the row's last token)
 *   row_qsl             device int32 [num_rows + 1]: row r's tokens are the
 *                       query rows row_qsl[r] .. row_qsl[r + 1] - 1, at most
 *                       pa_prefill_block_tokens of them (tokens past that
 *                       leave their outputs undefined)
 *   work_items          device int32 [num_rows][2], may be NULL: launch order,
 *                       (row, 0) for every row once, e.g. pa_prefill_plan
 *                       (a sequence's rows together, the largest sequences
 *                       first); NULL = the last row first, so that a
 *                       sequence's rows run together
 *   max_context_len     host bound on row_lens, checked against bt_stride
 *   sliding_window      as for pa_paged_attention_multi
 * Every key a row sees, its own new tokens included, must already be in the
 * caches (pa_reshape_and_cache before this call).  Errors: as
 * pa_paged_attention_multi's checks of sizes, pointers and alignment, plus
 * PA_EINVAL for f32 storage, head_size 64, null row arrays, num_rows < 1 or
 * a scale that is not positive and finite.
 * ---------------------------------------------------------------------- */
int32_t pa_prefill_block_tokens(int32_t num_heads, int32_t num_kv_heads, int32_t* tokens);

int32_t pa_paged_attention_prefill(void* out, const void* query, const void* key_cache,
                                   const void* value_cache, const int32_t* block_tables,
                                   int64_t bt_stride, const int32_t* row_seq,
                                   const int32_t* row_lens, const int32_t* row_qsl,
                                   int32_t num_rows, int32_t num_heads, int32_t num_kv_heads,
                                   int32_t head_size, int32_t block_size,
                                   int32_t max_context_len, float scale, int32_t dtype,
                                   const int32_t* work_items, int32_t sliding_window,
                                   void* stream);

/* pa_paged_attention_prefill_split: pa_paged_attention_prefill with the keys
 * of each row cut into partitions of partition_size, for batches with too
 * few (row, KV head) workgroups to fill the GPU (a long context under few
 * rows).  One workgroup per (work item, KV head) attends partition p of row
 * r and writes each of the row's query vectors' partial (m, l, o) to the
 * split workspace, as pa_paged_attention_decode_split's partition kernel
 * does; a merge launch then combines the partitions of each new token (those
 * below the row's length, from the token's window on) into out: the split-K
 * partition/merge described above (not in the pages), with the prefill
 * kernel's tiles.
 *   work_items      device int32 [num_work_items][2]: (row, p) pairs, every
 *                   partition of every row that holds a key one of its
 *                   tokens sees (pa_prefill_plan_split lists exactly those);
 *                   a missing item leaves the outputs that need it undefined,
 *                   a p at or past ceil(max_context_len / partition_size)
 *                   writes nothing
 *   partition_size  a multiple of 16 and of block_size, at most 4096
 *   workspace       device, 256-byte aligned, at least pa_split_workspace_bytes(
 *                   num_tokens, num_heads, head_size, max_context_len,
 *                   partition_size) bytes (num_tokens = row_qsl[num_rows]:
 *                   one workspace row per new token)
 * The other arguments and the requirements on the caches are those of
 * pa_paged_attention_prefill; the step's cache writes go first (there is no
 * one-launch form with partitions).  Errors: as pa_paged_attention_prefill,
 * plus PA_EINVAL for a null or empty work list, a bad partition_size,
 * num_tokens outside [1, 2^31), or a missing, small or misaligned workspace. */
int32_t pa_paged_attention_prefill_split(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, int64_t bt_stride, const int32_t* row_seq,
    const int32_t* row_lens, const int32_t* row_qsl, int32_t num_rows, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_size, int32_t block_size, int32_t max_context_len,
    float scale, int32_t dtype, const int32_t* work_items, int64_t num_work_items,
    int32_t partition_size, int32_t sliding_window, void* workspace, size_t workspace_bytes,
    int64_t num_tokens, void* stream);

/* ------------------------------------------------------------------------
 * pa_prefill_step: pa_paged_attention_prefill with the step's cache writes
 * in the same launch (the prefill counterpart of pa_decode_step): the
 * copy-on-write of the old slots of each fresh tail block, the new tokens'
 * K/V rows into their slots, and their slots into slot_mapping.  The
 * attention reads keys from a sequence's first new position on from the
 * key/value rows and the old slots of a copied tail from its source block,
 * so no workgroup reads a slot the launch writes, and the result is that of
 * the separate calls (copy_blocks, compute_slot_mapping, reshape_and_cache,
 * pa_paged_attention_prefill), bit for bit, in out, slot_mapping and every
 * cache slot below a sequence's length.  The slots at or past that length
 * of a copied block, which copy_blocks fills from the source block, are left
 * unspecified.
 *   query_start_loc  device int32 [num_seqs + 1]: sequence s's new tokens are
 *                    the rows query_start_loc[s] .. [s + 1] - 1 of query, key
 *                    and value; row_seq indexes these sequences and row_qsl
 *                    the same token rows
 *   key, value       device [num_tokens][...], rows key_stride / value_stride
 *                    elements apart (>= num_kv_heads * head_size, 16-byte
 *                    aligned), head kvh at kvh * head_size
 *   cow_src          device int64 [num_seqs]: the block whose first slots
 *                    sequence s's last block copies, or -1; NULL = none
 *   slot_mapping     device int64 [num_tokens] output, or NULL
 * block_tables must hold each sequence's blocks after the step's
 * allocation.  Errors: those of pa_paged_attention_prefill, plus PA_EINVAL
 * for a NULL query_start_loc, key or value, misaligned rows or strides, and
 * strides of 2^35 bytes or more.
 * ---------------------------------------------------------------------- */
int32_t pa_prefill_step(void* out, const void* query, void* key_cache, void* value_cache,
                        const int32_t* block_tables, int64_t bt_stride, const int32_t* row_seq,
                        const int32_t* row_lens, const int32_t* row_qsl, int32_t num_rows,
                        int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                        int32_t block_size, int32_t max_context_len, float scale, int32_t dtype,
                        const int32_t* work_items, int32_t sliding_window,
                        const int32_t* query_start_loc, const void* key, const void* value,
                        int64_t key_stride, int64_t value_stride, const int64_t* cow_src,
                        int64_t* slot_mapping, void* stream);

/* ------------------------------------------------------------------------
 * Attention alone over a cascade plan (pa_decode_plan_cascade), on caches that
 * already hold the step's rows: pa_paged_attention_decode_planned's
 * arguments, with the plan (device int32, whole: items and group section),
 * its num_items and max_group_size (its max_members) in place of the work
 * list.  partition_size == 0: single pass, workspace may be NULL;
 * partition_size > 0: partition kernel plus merge, workspace as for
 * pa_paged_attention_decode_split.  Same requirements and errors as
 * pa_decode_step_cascade, without its cache-write arguments.
 * ---------------------------------------------------------------------- */
int32_t pa_paged_attention_cascade(void* out, const void* query, const void* key_cache,
                                   const void* value_cache, const int32_t* block_tables,
                                   int64_t bt_stride, const int32_t* context_lens,
                                   int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                   int32_t head_size, int32_t block_size,
                                   int32_t max_context_len, float scale, int32_t dtype,
                                   int32_t partition_size, const int32_t* plan,
                                   int64_t num_items, int32_t max_group_size, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Several new tokens per sequence (speculative drafts, short prefill chunks;
 * [CSDN] section 2.3 lays a step's tokens out by query_start_loc, [DEEPSONAR]
 * section 2.5 schedules them like decode tokens).  Sequence s has n_s =
 * query_start_loc[s+1] - query_start_loc[s] new tokens, the last n_s of its
 * context_lens[s] tokens (already in the cache); new token i (row
 * query_start_loc[s] + i, position L_s - n_s + i) attends to positions
 * 0 .. L_s - n_s + i: the whole earlier context and the new tokens up to
 * itself.  n_s = 1 everywhere is the decode call.
 *   out, query       device [num_tokens][num_heads][head_size]
 *   query_start_loc  device int32 [num_seqs + 1], from 0 to num_tokens
 *   max_query_len    host bound on n_s; max_query_len x (num_heads /
 *                    num_kv_heads) must be at most 16 for 16-bit storage and
 *                    head_size 128 (matrix-core kernel), else at most 8
 *   workspace        split-K only: pa_split_workspace_bytes(num_tokens, ...)
 * Work items, shared_prefix_blocks, partition_size and sliding_window as in
 * pa_paged_attention_decode_planned (items are (sequence, partition), from
 * pa_decode_plan_window with the query lengths when a window is used).
 * ---------------------------------------------------------------------- */
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
                                 int32_t sliding_window, void* stream);

/* ------------------------------------------------------------------------
 * Host block allocator (CPU memory only; no device calls).  Generates the
 * block tables, slots and copy-on-write pairs the kernels consume.
 *   [PUFANYI] "按 Block 分配": a sequence of T tokens holds ceil(T/B)
 *   blocks; new tokens fill the tail block first, a fresh block is taken
 *   only when the tail is full.
 *   [CSDN] section 3.2.1: fresh blocks come from the head of the free queue;
 *   a request that does not fit fails without side effects.
 *   [CSDN] sections 3.1.2 and 3.2.4: a released request drops its blocks
 *   tail first; blocks whose count reaches 0 join the tail of the queue.
 *   [CSDN] section 3.2.3 (touch) and [VLLBC] paper section 4.4 / Fig. 8:
 *   sharing raises per-block reference counts; a writer whose partly filled
 *   tail is shared copies it to a fresh block first (copy-on-write); the
 *   last holder writes in place.
 * The free queue starts in the caller's order (initial_free_order, a
 * permutation of 0..num_blocks-1; NULL means ascending).  Sequences are
 * named by caller-chosen int64 ids.  A pool is not thread-safe.
 * ---------------------------------------------------------------------- */
typedef struct pa_pool pa_pool;

/* Create a pool. *out receives the handle. PA_EINVAL for sizes < 1 or an
 * initial order that is not a permutation. */
int32_t pa_pool_create(int32_t num_blocks, int32_t block_size,
                       const int32_t* initial_free_order, pa_pool** out);
/* Destroy a pool (NULL is ignored). */
void pa_pool_destroy(pa_pool* pool);
/* Register an empty sequence. PA_EINVAL if the id exists. */
int32_t pa_pool_add_seq(pa_pool* pool, int64_t seq);
/* child shares every block of parent (each count + 1) and its length.
 * PA_EINVAL if parent is unknown or child exists. */
int32_t pa_pool_fork(pa_pool* pool, int64_t parent, int64_t child);
/* Append n >= 1 tokens to seq.  slots_out (host int64 [n]) receives the
 * physical slot of each new token; cow_pair_out (host int64 [2], may be NULL
 * only if the caller knows no copy can happen) receives (src, dst) when the
 * shared tail was copied, and *n_cow_out (0 or 1) says whether it was.
 * All-or-nothing: PA_ENOMEM leaves the pool unchanged. */
int32_t pa_pool_append(pa_pool* pool, int64_t seq, int32_t n, int64_t* slots_out,
                       int64_t* cow_pair_out, int32_t* n_cow_out);
/* Release seq: counts drop tail first; blocks reaching 0 join the queue tail. */
int32_t pa_pool_free_seq(pa_pool* pool, int64_t seq);
/* Length (tokens) and number of blocks held by seq. */
int32_t pa_pool_seq_len(const pa_pool* pool, int64_t seq, int64_t* len_out);
int32_t pa_pool_seq_num_blocks(const pa_pool* pool, int64_t seq, int32_t* n_out);
/* Block tables of num_seqs sequences into host int32 out[num_seqs][width],
 * unused entries -1; context_lens_out (host int32 [num_seqs], may be NULL)
 * receives the lengths.  PA_EINVAL if a sequence holds more than width
 * blocks or is unknown. */
int32_t pa_pool_block_tables(const pa_pool* pool, const int64_t* seqs, int32_t num_seqs,
                             int32_t* out, int32_t width, int32_t* context_lens_out);
/* For each of num_seqs sequences, the number of leading blocks of its table
 * whose reference count is above 1 (blocks other sequences share), into
 * host int32 out[num_seqs]; released entries (-1) may sit inside that
 * prefix, which ends after its last shared block.  PA_EINVAL for an unknown
 * sequence. */
int32_t pa_pool_shared_prefix_blocks(const pa_pool* pool, const int64_t* seqs, int32_t num_seqs,
                                     int32_t* out);
/* Number of free blocks; reference count of one block (-1 if out of range). */
int32_t pa_pool_num_free(const pa_pool* pool);
int32_t pa_pool_ref(const pa_pool* pool, int32_t block);
/* Free queue from head to tail into host int32 out[cap]; returns the count
 * written, or -1 on a null argument. */
int32_t pa_pool_free_queue(const pa_pool* pool, int32_t* out, int32_t cap);
/* Number of copy-on-write copies performed since creation. */
int64_t pa_pool_num_cow(const pa_pool* pool);
/* Sliding window ([CSDN] sections 3.1.1 and 3.3.1: before allocating, the
 * blocks outside the window are released).  With num_computed_tokens N
 * computed, the next query (position N) sees positions N - W + 1 .. N (the
 * reading pa_paged_attention_decode_planned documents), so
 * max(0, N - W + 1) tokens are skipped and the first floor of that over B
 * blocks of seq are released: tail first, counts down, blocks reaching 0 to
 * the queue tail.  Their table entries become -1 (pa_pool_block_tables
 * reports them; windowed attention never reads them); the length is
 * unchanged.  sliding_window == 0 releases nothing.  *num_released (may be
 * NULL) receives how many blocks this call released.  PA_EINVAL for an
 * unknown sequence or a negative argument. */
int32_t pa_pool_remove_skipped(pa_pool* pool, int64_t seq, int64_t num_computed_tokens,
                               int32_t sliding_window, int32_t* num_released);
/* The appends of one step, as a whole or not at all ([CSDN] section 3.2.1:
 * a request that does not fit is refused without side effects; sections
 * 3.1.1 and 3.3.1: blocks outside the window are released before the
 * allocation; section 3.4: the kernels' smaller blocks).  Row r appends
 * num_new[r] tokens to seqs[r]: with sliding_window > 0 it first releases
 * what its next query no longer sees (pa_pool_remove_skipped at its current
 * length), then appends (pa_pool_append), rows in order.
 * Before anything changes, every row is checked (a known sequence, listed
 * once, num_new >= 1) and the free queue is followed through the rows in
 * order, counting the blocks earlier rows release, copy and take: PA_EINVAL
 * or PA_ENOMEM then leave the pool exactly as it was.
 * Outputs (host buffers; T = the sum of num_new, k = blocks_per_kv_block,
 * 1 when the allocator's blocks are the kernels' blocks):
 *   positions_out        int64 [T]: position of each new token, rows in order
 *   query_start_loc_out  int32 [num_seqs + 1]: row r's tokens are
 *                        [qsl[r], qsl[r+1])
 *   slots_out            int64 [T] or NULL: slot of each new token (the same
 *                        number under manager and kernel blocks)
 *   cow_src_out          int64 [num_seqs]: the manager block row r's shared
 *                        tail was copied from, -1 if none
 *   cow_pairs_out        int64 [num_seqs * k][2]: the copies for
 *                        pa_copy_blocks in kernel blocks: manager pair
 *                        (src, dst) gives (src*k + j, dst*k + j), j < k
 *   num_cow_pairs_out    number of pairs written
 *   shared_blocks_out    int32 [num_seqs] or NULL: after the appends, the
 *                        leading shared blocks of each table
 *                        (pa_pool_shared_prefix_blocks) in kernel blocks
 *   group_keys_out       int32 [num_seqs] or NULL: a key for
 *                        pa_decode_plan_window that rows reading the same
 *                        shared prefix have in common (its first live kernel
 *                        block); a row without shared blocks gets
 *                        num_blocks * k + r.
 * PA_EINVAL also for null required pointers, num_seqs < 1, a negative
 * window, k < 1 or kernel block ids past int32. */
int32_t pa_pool_append_batch(pa_pool* pool, const int64_t* seqs, const int32_t* num_new,
                             int32_t num_seqs, int32_t sliding_window,
                             int32_t blocks_per_kv_block, int64_t* positions_out,
                             int32_t* query_start_loc_out, int64_t* slots_out,
                             int64_t* cow_src_out, int64_t* cow_pairs_out,
                             int32_t* num_cow_pairs_out, int32_t* shared_blocks_out,
                             int32_t* group_keys_out);

/* ------------------------------------------------------------------------
 * Prefix caching on the host ([DEEPSONAR] section 2.4; [CSDN] sections
 * 3.2.1-3.2.3, 5.2 and 5.3; [PUFANYI] "共享前缀，分叉时 Copy-on-write").
 * Every full block of a request is keyed by a chained SHA-256 over the
 * parent block's key, the block's token ids and the request's extra key
 * bytes (e.g. an adapter id), so equal keys mean equal whole prefixes.
 * Message layout (this library's reading; the pages name the three inputs
 * only): parent key (32 bytes) || token ids as little-endian int32 ||
 * extra bytes; the first block's parent key is 32 zero bytes.
 *
 * A new request takes over its longest run of cached blocks from the start
 * of its prompt, stopping at the first key that is not cached and at
 * (prompt length - 1) / B blocks: the last prompt token is always computed
 * again.  Taken-over blocks gain a holder (one with none leaves the free
 * queue).  Freed cached blocks keep their key while they wait in the free
 * queue, which is the LRU order: a block taken from its head for new tokens
 * loses its key (eviction).  A key already held by another block keeps that
 * block.
 *
 * pa_pool_enable_prefix_caching: switch the cache on; only before the first
 *   sequence.  PA_EINVAL otherwise.
 * pa_pool_add_seq_cached: new sequence for a prompt of host int32 token ids;
 *   *num_computed_tokens receives how many prompt tokens came from the cache
 *   (a multiple of B); the caller appends the rest with
 *   pa_pool_append_tokens.  PA_EINVAL when caching is off, the sequence
 *   exists or an argument is bad.
 * pa_pool_append_tokens: pa_pool_append that also records the token ids
 *   (host int32 [n]); plain pa_pool_append stops a sequence's recording and
 *   then pa_pool_cache_full_blocks refuses it.
 * pa_pool_cache_full_blocks: key every full block of seq that has no key yet
 *   (after its K/V were written); *num_cached (may be NULL) receives how many
 *   blocks were added to the cache.
 * pa_pool_num_cached_blocks / pa_pool_num_evicted: cache size and evictions
 *   so far (-1 for a null pool).
 * pa_block_keys (host only): the key chain of a token sequence, 32 bytes per
 *   full block into keys_out [num_tokens / block_size][32].
 * ---------------------------------------------------------------------- */
int32_t pa_pool_enable_prefix_caching(pa_pool* pool);
int32_t pa_pool_add_seq_cached(pa_pool* pool, int64_t seq, const int32_t* prompt,
                               int64_t num_prompt_tokens, const void* extra,
                               int32_t extra_bytes, int64_t* num_computed_tokens);
int32_t pa_pool_append_tokens(pa_pool* pool, int64_t seq, const int32_t* tokens, int32_t n,
                              int64_t* slots_out, int64_t* cow_pair_out, int32_t* n_cow_out);
int32_t pa_pool_cache_full_blocks(pa_pool* pool, int64_t seq, int32_t* num_cached);
int64_t pa_pool_num_cached_blocks(const pa_pool* pool);
int64_t pa_pool_num_evicted(const pa_pool* pool);
int32_t pa_block_keys(const int32_t* tokens, int64_t num_tokens, int32_t block_size,
                      const void* extra, int32_t extra_bytes, uint8_t* keys_out);

/* Kernel blocks ([CSDN] section 3.4, hybrid block sizes): when the
 * allocator's blocks hold k = blocks_per_kv_block smaller blocks of the
 * kernels, manager block b stands for kernel blocks b*k .. b*k + k - 1.
 * Host only: kernel_ids (host int32 [n * k]) receives the mapping of
 * manager_ids (host int32 [n]); -1 entries map to k entries of -1.  The
 * kernels then take the mapped table with block size B / k and a cache of
 * num_blocks * k kernel blocks [..][num_kv_heads][B / k][head_size]; slot
 * numbers are the same under both tables.  Copy-on-write pairs map the same
 * way, pair by pair.  PA_EINVAL for null pointers with n > 0, n < 0,
 * blocks_per_kv_block < 1 or an id whose kernel ids overflow int32 (then
 * nothing is written). */
int32_t pa_map_to_kernel_blocks(const int32_t* manager_ids, int64_t n,
                                int32_t blocks_per_kv_block, int32_t* kernel_ids);

/* ------------------------------------------------------------------------
 * Attention partials and their merge (context parallelism, [CSDN] section
 * 2.3).  Each rank attends over the tokens it stores and keeps, per
 * (sequence, query head), m = max of the scaled scores x_t (natural log
 * domain), l = sum exp(x_t - m) and o = sum exp(x_t - m) v_t / l; gathering
 * the ranks' (m, l, o) and merging them with M = max m_r,
 * a_r = l_r exp(m_r - M), out = sum a_r o_r / sum a_r gives attention over
 * the whole context (the split-K merge over ranks instead of partitions).
 * The exchange between ranks is the caller's (an all-gather of
 * head_size + 2 floats per (sequence, query head)).
 *
 * pa_paged_attention_partials: the rank-local (m, l, o), fp32.
 *   max_logits, exp_sums  device float [num_seqs][num_heads] (output)
 *   partial_out           device float [num_seqs][num_heads][head_size]
 *                         (output), 16-byte aligned
 *   context_lens          device int32 [num_seqs], rank-local lengths; 0 is
 *                         allowed and gives m = -inf, l = 0, o = 0
 *   max_context_len       >= 0, at least every context_lens entry
 *   partition_size        > 0, as pa_paged_attention_decode_split; the
 *                         partitions are merged inside the call
 *   work_items            NULL (one workgroup per (partition, KV head,
 *                         sequence)) or a pa_decode_plan list for this
 *                         partition_size
 *   workspace             as pa_paged_attention_decode_split for
 *                         max(max_context_len, 1); may be NULL when
 *                         max_context_len == 0
 *   Other arguments as pa_paged_attention_decode_planned.
 *
 * pa_merge_attention_partials: out [num_seqs][num_heads][head_size] in the
 * storage dtype from num_parts gathered sets, rank-major:
 *   max_logits, exp_sums  device float [num_parts][num_seqs][num_heads]
 *   partial_out           device float [num_parts][num_seqs][num_heads][head_size],
 *                         8-byte aligned
 * Parts with l = 0 carry no weight; a row no part has a key for is 0.
 * Errors: PA_EINVAL for null pointers, num_parts < 1, num_seqs < 1,
 * num_heads < 1, num_seqs x ceil(num_heads / 4) above INT32_MAX (the merge's
 * workgroups), head_size not 64 or 128, an unknown dtype, out not aligned to
 * its element size, partial_out not 8-byte aligned.
 * ---------------------------------------------------------------------- */
int32_t pa_paged_attention_partials(float* max_logits, float* exp_sums, float* partial_out,
                                    const void* query, const void* key_cache,
                                    const void* value_cache, const int32_t* block_tables,
                                    int64_t bt_stride, const int32_t* context_lens,
                                    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                    int32_t head_size, int32_t block_size,
                                    int32_t max_context_len, float scale, int32_t dtype,
                                    int32_t partition_size, const int32_t* work_items,
                                    int64_t num_work_items, const int32_t* shared_prefix_blocks,
                                    void* workspace, size_t workspace_bytes, void* stream);

int32_t pa_merge_attention_partials(void* out, const float* max_logits, const float* exp_sums,
                                    const float* partial_out, int32_t num_parts,
                                    int32_t num_seqs, int32_t num_heads, int32_t head_size,
                                    int32_t dtype, void* stream);

/* ------------------------------------------------------------------------
 * Diagnostic (not part of the decode path): reads num_blocks whole 4 KiB
 * blocks of buffer, block block_order[i] for i = 0..num_blocks-1, with `grid`
 * workgroups of 256 lanes x 16 bytes, as non-temporal loads when
 * non_temporal != 0.  A reference of achievable read
 * bandwidth for a given block order, and a kernel of known byte count for
 * calibrating hardware counters.
 *   buffer       device, 16-byte aligned, >= 4096 * (max(block_order) + 1) bytes
 *   block_order  device int32 [num_blocks], each in range (trusted)
 *   sink         device, >= 4 bytes (written only on a one-in-2^32 value)
 * Errors: PA_EINVAL for null pointers, num_blocks < 1, grid < 1, alignment.
 * ---------------------------------------------------------------------- */
int32_t pa_probe_read_blocks(const void* buffer, const int32_t* block_order, int64_t num_blocks,
                             void* sink, int32_t grid, int32_t non_temporal, void* stream);

/* ------------------------------------------------------------------------
 * Diagnostic (not part of the decode path): a per-workgroup timeline of the
 * single-pass cascade kernel, recorded only by a library built with
 * PA_TIMELINE=1 (python -m paged_kv_cache_123_amd.build -D PA_TIMELINE=1
 * --out PATH); the default build returns PA_EINVAL from both calls.
 * Workgroup i < 8192 of the last cascade launch writes record i: four
 * uint64 words, the GPU real-time counter (100 MHz, one clock for every CU)
 * at its entry, when its first round of tiles has been described, and at
 * its exit, then (XCC id << 32) | HW_ID register (CU, SIMD and wave slot of
 * its first wave).  Concurrent cascade launches overwrite each other's
 * records.
 *   pa_timeline_reset: clears the records (asynchronous on stream).
 *   pa_timeline_read: copies min(capacity, 8192) records to host memory
 *     (records: host uint64 [4 * capacity]; synchronous) and sets
 *     *num_records to the number of leading records written since the reset.
 * Errors: PA_EINVAL for a default build, null pointers or capacity < 1;
 * PA_ELAUNCH when the clear or the copy fails.
 * ---------------------------------------------------------------------- */
int32_t pa_timeline_reset(void* stream);
int32_t pa_timeline_read(uint64_t* records, int64_t capacity, int64_t* num_records);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
