// Host-side work plan for the attention calls: every non-empty (sequence,
// partition) pair once, largest first, so that workgroups of a launch start
// in decreasing order of work and none is launched without work.  Sizes are
// compared in buckets of kGranule tokens and equal buckets keep batch order,
// so sequences that share blocks (forks of one prompt sit next to each other
// in a batch) still run close together in time and reuse cached blocks.
// With a sliding window an item's size is the part of it inside the window,
// and partitions wholly before the window are left out.  Group keys (e.g. the
// first block of a shared prefix) order the items of one bucket by group, so
// the readers of one prefix run together wherever they sit in the batch.
#include <algorithm>
#include <climits>
#include <cstdint>
#include <map>
#include <string>
#include <vector>

#include "pagedkv.h"
#include "status.h"

namespace {
constexpr int32_t kGranule = 256;
constexpr int32_t kTileTokens = 16;  // keys per tile of the cascade kernel
}

extern "C" int32_t pa_decode_plan_window(const int32_t* context_lens,
                                         const int32_t* query_lens, const int32_t* group_keys,
                                         int32_t num_seqs, int32_t partition_size,
                                         int32_t sliding_window, int32_t* items,
                                         int64_t capacity, int64_t* num_items) {
  if (!context_lens || !num_items || num_seqs < 1 || partition_size < 0 || sliding_window < 0)
    return pa::fail(PA_EINVAL, "pa_decode_plan: bad argument");
  struct Item {
    int32_t tokens, group, s, p;
  };
  std::vector<Item> v;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t L = context_lens[s];
    if (L < 0 || (L == 0 && partition_size == 0))
      return pa::fail(PA_EINVAL, "pa_decode_plan: context length < 1");
    const int32_t n = query_lens ? query_lens[s] : 1;
    if (L > 0 && (n < 1 || n > L))
      return pa::fail(PA_EINVAL, "pa_decode_plan: query length outside [1, context length]");
    // first key the sequence's first query sees under the window
    const int32_t lo = sliding_window > 0 ? std::max(0, L - n + 1 - sliding_window) : 0;
    // sequences with one group key (readers of one shared prefix) run together
    const int32_t g = group_keys ? group_keys[s] : s;
    if (partition_size == 0) {
      v.push_back({L - lo, g, s, 0});
      continue;
    }
    // a sequence with no token (a rank-local share can be empty) has no item;
    // partitions wholly before the window have none either
    for (int32_t p = lo / partition_size; static_cast<int64_t>(p) * partition_size < L; ++p) {
      const int32_t begin = std::max(p * partition_size, lo);
      v.push_back({std::min((p + 1) * partition_size, L) - begin, g, s, p});
    }
  }
  *num_items = static_cast<int64_t>(v.size());
  if (!items) return PA_OK;  // size query
  if (capacity < static_cast<int64_t>(v.size()))
    return pa::fail(PA_EINVAL, "pa_decode_plan: capacity smaller than the number of items");
  std::stable_sort(v.begin(), v.end(), [](const Item& a, const Item& b) {
    const int32_t ba = (a.tokens + kGranule - 1) / kGranule;
    const int32_t bb = (b.tokens + kGranule - 1) / kGranule;
    return ba != bb ? ba > bb : a.group < b.group;
  });
  for (size_t i = 0; i < v.size(); ++i) {
    items[2 * i] = v[i].s;
    items[2 * i + 1] = v[i].p;
  }
  return PA_OK;
}

extern "C" int32_t pa_decode_plan(const int32_t* context_lens, int32_t num_seqs,
                                  int32_t partition_size, int32_t* items, int64_t capacity,
                                  int64_t* num_items) {
  return pa_decode_plan_window(context_lens, nullptr, nullptr, num_seqs, partition_size, 0,
                               items, capacity, num_items);
}

// Cascade plan: the partitions that lie wholly inside a prefix several
// sequences share are computed once per group of sharers instead of once per
// sequence.  Sequences are candidates for one group when their first table
// entry is the same block; the group's prefix is the run of leading table
// entries all members agree on, cut to full blocks that end before any
// member's first new token (no row of it is written during the step).  A
// group is split into chunks of at most max_group_size members; chunk c and
// partition p (wholly inside the prefix) make the item (-1 - c, p).  Every
// other (sequence, partition) pair keeps its own item.
// With partition_size == 0 (single pass) a chunk's item is (-1 - c, prefix
// tokens): one workgroup per KV head reads the prefix once for all members
// and then every member's own tokens past it; every other sequence s keeps
// the item (s, 0).  Items are ordered by the tokens they read.  Layout of
// `plan`:
//   [2 * num_items]           the items, largest first as in pa_decode_plan
//   [1]                       number of chunks C
//   [C + 1]                   offsets of each chunk's members
//   [offsets[C]]              members (batch rows), in batch order per chunk
namespace {

// Groups of sharers, as both cascade plans form them: sequences whose first
// table entry is the same block are candidates; the group's prefix is the run
// of leading entries all of them agree on, cut to full blocks that end before
// any member's first new token; a group is split into chunks of at most
// max_group_size members (a lone member is left out).
struct CascadeGroups {
  std::vector<int32_t> off{0};   // chunk c's members: members[off[c] .. off[c+1])
  std::vector<int32_t> members;  // batch rows
  std::vector<int32_t> prefix;   // shared prefix tokens of each chunk
  std::vector<uint8_t> grouped;  // per sequence: in a chunk
};

int32_t form_groups(const char* who, const int32_t* context_lens, const int32_t* block_tables,
                    int64_t bt_stride, const int32_t* new_tokens, int32_t num_seqs,
                    int32_t block_size, int32_t max_group_size, CascadeGroups& g) {
  std::vector<int32_t> first_new(num_seqs);
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t L = context_lens[s];
    const int32_t n = new_tokens ? new_tokens[s] : 1;
    if (L < 1 || n < 1 || n > L)
      return pa::fail(PA_EINVAL,
                      (std::string(who) + ": need 1 <= new tokens <= context length").c_str());
    if ((static_cast<int64_t>(L) + block_size - 1) / block_size > bt_stride)
      return pa::fail(PA_EINVAL, (std::string(who) + ": table row shorter than the length").c_str());
    first_new[s] = L - n;
  }
  auto row = [&](int32_t s) { return block_tables + static_cast<int64_t>(s) * bt_stride; };
  std::vector<int32_t> order(num_seqs);
  for (int32_t s = 0; s < num_seqs; ++s) order[s] = s;
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t a, int32_t b) { return row(a)[0] < row(b)[0]; });
  g.grouped.assign(num_seqs, 0);
  for (size_t i = 0; i < order.size();) {
    size_t j = i + 1;
    while (j < order.size() && row(order[j])[0] == row(order[i])[0]) ++j;
    if (j - i >= 2 && row(order[i])[0] >= 0) {
      int32_t limit = INT32_MAX;
      for (size_t k = i; k < j; ++k) limit = std::min(limit, first_new[order[k]] / block_size);
      int32_t common = 0;
      while (common < limit) {
        const int32_t b = row(order[i])[common];
        bool same = b >= 0;
        for (size_t k = i + 1; k < j && same; ++k) same = row(order[k])[common] == b;
        if (!same) break;
        ++common;
      }
      if (common > 0) {
        std::vector<int32_t> grp(order.begin() + i, order.begin() + j);
        std::sort(grp.begin(), grp.end());
        for (size_t c = 0; c < grp.size(); c += max_group_size) {
          const size_t e = std::min(grp.size(), c + max_group_size);
          if (e - c < 2) break;  // a lone member keeps its own items
          for (size_t k = c; k < e; ++k) {
            g.members.push_back(grp[k]);
            g.grouped[grp[k]] = 1;
          }
          g.off.push_back(static_cast<int32_t>(g.members.size()));
          g.prefix.push_back(common * block_size);
        }
      }
    }
    i = j;
  }
  return PA_OK;
}

struct PlanItem {
  int32_t tokens, key, s, p;
};

// Items largest first (by tokens read, in buckets), then the plan's group
// section: C, the C + 1 member offsets, optionally the C prefix lengths, the
// members.
int32_t write_plan(const char* who, std::vector<PlanItem>& v, const CascadeGroups& g,
                   bool with_prefix, int32_t granule, int32_t* plan, int64_t capacity,
                   int64_t* num_items, int64_t* plan_len, int32_t* max_members) {
  const int32_t num_chunks = static_cast<int32_t>(g.prefix.size());
  int32_t widest = 0;
  for (int32_t c = 0; c < num_chunks; ++c) widest = std::max(widest, g.off[c + 1] - g.off[c]);
  *num_items = static_cast<int64_t>(v.size());
  *plan_len = 2 * static_cast<int64_t>(v.size()) + 1 + (num_chunks + 1) +
              (with_prefix ? num_chunks : 0) + static_cast<int64_t>(g.members.size());
  *max_members = widest;
  if (!plan) return PA_OK;  // size query
  if (capacity < *plan_len)
    return pa::fail(PA_EINVAL, (std::string(who) + ": capacity smaller than the plan").c_str());
  std::stable_sort(v.begin(), v.end(), [granule](const PlanItem& a, const PlanItem& b) {
    const int32_t ba = (a.tokens + granule - 1) / granule;
    const int32_t bb = (b.tokens + granule - 1) / granule;
    return ba != bb ? ba > bb : a.key < b.key;
  });
  int64_t w = 0;
  for (const PlanItem& it : v) {
    plan[w++] = it.s;
    plan[w++] = it.p;
  }
  plan[w++] = num_chunks;
  for (int32_t o : g.off) plan[w++] = o;
  if (with_prefix)
    for (int32_t t : g.prefix) plan[w++] = t;
  for (int32_t m : g.members) plan[w++] = m;
  return PA_OK;
}

}  // namespace

// Cascade plan: the partitions that lie wholly inside a prefix several
// sequences share are computed once per group of sharers instead of once per
// sequence (groups as form_groups makes them).  Chunk c and partition p
// (wholly inside the prefix) make the item (-1 - c, p).  Every other
// (sequence, partition) pair keeps its own item.
// With partition_size == 0 (single pass) a chunk's item is (-1 - c, prefix
// tokens): one workgroup per KV head reads the prefix once for all members
// and then every member's own tokens past it; every other sequence s keeps
// the item (s, 0).  Items are ordered by the tokens they read.  Layout of
// `plan`:
//   [2 * num_items]           the items, largest first as in pa_decode_plan
//   [1]                       number of chunks C
//   [C + 1]                   offsets of each chunk's members
//   [offsets[C]]              members (batch rows), in batch order per chunk
extern "C" int32_t pa_decode_plan_cascade(const int32_t* context_lens,
                                          const int32_t* block_tables, int64_t bt_stride,
                                          const int32_t* new_tokens, int32_t num_seqs,
                                          int32_t block_size, int32_t partition_size,
                                          int32_t max_group_size, int32_t* plan,
                                          int64_t capacity, int64_t* num_items,
                                          int64_t* plan_len, int32_t* max_members) {
  const char* who = "pa_decode_plan_cascade";
  if (!context_lens || !block_tables || !num_items || !plan_len || !max_members ||
      num_seqs < 1 || block_size < 1 || partition_size < 0 || max_group_size < 1 ||
      partition_size % block_size != 0 || bt_stride < 1)
    return pa::fail(PA_EINVAL, "pa_decode_plan_cascade: bad argument");
  CascadeGroups g;
  int32_t st = form_groups(who, context_lens, block_tables, bt_stride, new_tokens, num_seqs,
                           block_size, max_group_size, g);
  if (st != PA_OK) return st;
  const bool single = partition_size == 0;
  // split plans keep only chunks with a whole partition inside the prefix
  if (!single) {
    CascadeGroups kept;
    kept.grouped.assign(num_seqs, 0);
    for (size_t c = 0; c + 1 < g.off.size(); ++c) {
      if (g.prefix[c] / partition_size == 0) continue;
      for (int32_t k = g.off[c]; k < g.off[c + 1]; ++k) {
        kept.members.push_back(g.members[k]);
        kept.grouped[g.members[k]] = 1;
      }
      kept.off.push_back(static_cast<int32_t>(kept.members.size()));
      kept.prefix.push_back(g.prefix[c]);
    }
    g = std::move(kept);
  }
  std::vector<PlanItem> v;
  const int32_t num_chunks = static_cast<int32_t>(g.prefix.size());
  for (int32_t c = 0; c < num_chunks; ++c) {
    if (single) {  // the prefix once, then each member's own tokens
      // (counted in the kernel's 16-token tiles: a member's last tile costs
      // a whole one)
      const int32_t prefix = g.prefix[c];
      int64_t tokens = (prefix + kTileTokens - 1) / kTileTokens * kTileTokens;
      for (int32_t k = g.off[c]; k < g.off[c + 1]; ++k)
        tokens += (context_lens[g.members[k]] - prefix + kTileTokens - 1) / kTileTokens *
                  kTileTokens;
      v.push_back({static_cast<int32_t>(std::min<int64_t>(tokens, INT32_MAX)),
                   g.members[g.off[c]], -1 - c, prefix});
      continue;
    }
    for (int32_t p = 0; p < g.prefix[c] / partition_size; ++p)
      v.push_back({partition_size, g.members[g.off[c]], -1 - c, p});
  }
  // split: a member's own items start after its chunk's prefix partitions
  std::vector<int32_t> own_from(num_seqs, 0);
  if (!single)
    for (int32_t c = 0; c < num_chunks; ++c)
      for (int32_t k = g.off[c]; k < g.off[c + 1]; ++k)
        own_from[g.members[k]] = g.prefix[c] / partition_size;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t L = context_lens[s];
    if (single) {
      if (!g.grouped[s]) v.push_back({L, s, s, 0});
      continue;
    }
    for (int32_t p = own_from[s]; static_cast<int64_t>(p) * partition_size < L; ++p)
      v.push_back({std::min((p + 1) * partition_size, L) - p * partition_size, s, s, p});
  }
  // single pass: one round of workgroups, whose end is that of the longest
  // items, so those go first, ordered exactly (in the kernel's tiles)
  return write_plan(who, v, g, false, single ? kTileTokens : kGranule, plan, capacity, num_items,
                    plan_len, max_members);
}

// Chunk size of a step's cascade plan: a single-pass plan runs one
// workgroup per (item, KV head); when that is less than one round of the
// chip (kRoundWorkgroups, two per compute unit) and some prefix spans at
// least two pieces of kAutoChunk tokens, the chunked plan spreads the
// prefixes over more workgroups.  0: the single-pass plan.
extern "C" int32_t pa_cascade_auto_chunk(const int32_t* context_lens,
                                         const int32_t* block_tables, int64_t bt_stride,
                                         const int32_t* new_tokens, int32_t num_seqs,
                                         int32_t block_size, int32_t max_group_size,
                                         int32_t num_kv_heads, int32_t* chunk_tokens) {
  constexpr int64_t kRoundWorkgroups = 512;
  constexpr int32_t kAutoChunk = 2048;
  const char* who = "pa_cascade_auto_chunk";
  if (!context_lens || !block_tables || !chunk_tokens || num_seqs < 1 || block_size < 1 ||
      max_group_size < 1 || num_kv_heads < 1 || bt_stride < 1)
    return pa::fail(PA_EINVAL, "pa_cascade_auto_chunk: bad argument");
  *chunk_tokens = 0;
  CascadeGroups g;
  const int32_t st = form_groups(who, context_lens, block_tables, bt_stride, new_tokens,
                                 num_seqs, block_size, max_group_size, g);
  if (st != PA_OK) return st;
  int64_t items = static_cast<int64_t>(g.prefix.size());
  for (int32_t s = 0; s < num_seqs; ++s) items += g.grouped[s] ? 0 : 1;
  int32_t longest = 0;
  for (int32_t t : g.prefix) longest = std::max(longest, t);
  if (items * num_kv_heads < kRoundWorkgroups && longest >= 2 * kAutoChunk &&
      kAutoChunk % block_size == 0)
    *chunk_tokens = kAutoChunk;
  return PA_OK;
}

// Chunked cascade plan (single-pass kernel, split into pieces of at most
// chunk_tokens): a chunk's shared prefix is cut into chunk_tokens pieces, each
// an item (-1 - c, j) for j < pf = prefix / chunk_tokens that reads its piece
// once for all members; the item (-1 - c, pf) reads the rest of the prefix
// [pf * chunk_tokens, prefix) once for all members and then every member's
// own tokens.  A sequence outside every chunk has the items (s, p), tokens
// [p * chunk_tokens, min((p + 1) * chunk_tokens, L)).  Every item writes
// partials that a merge over ceil(L / chunk_tokens) parts per sequence
// finishes.  Layout as pa_decode_plan_cascade, with the C prefix lengths
// after the member offsets.
extern "C" int32_t pa_decode_plan_cascade_chunked(
    const int32_t* context_lens, const int32_t* block_tables, int64_t bt_stride,
    const int32_t* new_tokens, int32_t num_seqs, int32_t block_size, int32_t chunk_tokens,
    int32_t max_group_size, int32_t* plan, int64_t capacity, int64_t* num_items,
    int64_t* plan_len, int32_t* max_members) {
  const char* who = "pa_decode_plan_cascade_chunked";
  if (!context_lens || !block_tables || !num_items || !plan_len || !max_members ||
      num_seqs < 1 || block_size < 1 || chunk_tokens < 1 || max_group_size < 1 ||
      chunk_tokens % block_size != 0 || bt_stride < 1)
    return pa::fail(PA_EINVAL, "pa_decode_plan_cascade_chunked: bad argument");
  CascadeGroups g;
  const int32_t st = form_groups(who, context_lens, block_tables, bt_stride, new_tokens,
                                 num_seqs, block_size, max_group_size, g);
  if (st != PA_OK) return st;
  std::vector<PlanItem> v;
  const int32_t num_chunks = static_cast<int32_t>(g.prefix.size());
  for (int32_t c = 0; c < num_chunks; ++c) {
    const int32_t prefix = g.prefix[c], pf = prefix / chunk_tokens;
    const int32_t key = g.members[g.off[c]];
    for (int32_t j = 0; j < pf; ++j) v.push_back({chunk_tokens, key, -1 - c, j});
    int64_t tokens = prefix - static_cast<int64_t>(pf) * chunk_tokens;
    for (int32_t k = g.off[c]; k < g.off[c + 1]; ++k)
      tokens += context_lens[g.members[k]] - prefix;
    v.push_back({static_cast<int32_t>(std::min<int64_t>(tokens, INT32_MAX)), key, -1 - c, pf});
  }
  for (int32_t s = 0; s < num_seqs; ++s) {
    if (g.grouped[s]) continue;
    const int32_t L = context_lens[s];
    for (int32_t p = 0; static_cast<int64_t>(p) * chunk_tokens < L; ++p)
      v.push_back({std::min((p + 1) * chunk_tokens, L) - p * chunk_tokens, s, s, p});
  }
  return write_plan(who, v, g, true, kGranule, plan, capacity, num_items, plan_len, max_members);
}

// Query blocks: sequence s's n_s new tokens (rows [qsl[s], qsl[s+1]) of the
// step's queries, positions [L_s - n_s, L_s)) are cut into blocks of at most
// max_block tokens.  Block j becomes a row of its own for the multi-query
// attention: its tokens are rows [qsl[s] + j*max_block, ...) and it sees the
// sequence's positions up to its last token, so its context length is
// L_s - n_s + (end of the block) and its causal bounds are those of the
// tokens in the whole sequence.
extern "C" int32_t pa_query_blocks(const int32_t* context_lens, const int32_t* query_start_loc,
                                   int32_t num_seqs, int32_t max_block, int32_t* row_seq,
                                   int32_t* row_lens, int32_t* row_qsl, int64_t capacity,
                                   int64_t* num_rows) {
  if (!context_lens || !query_start_loc || !num_rows || num_seqs < 1 || max_block < 1)
    return pa::fail(PA_EINVAL, "pa_query_blocks: bad argument");
  int64_t rows = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t n = query_start_loc[s + 1] - query_start_loc[s];
    if (n < 1 || n > context_lens[s])
      return pa::fail(PA_EINVAL, "pa_query_blocks: need 1 <= new tokens <= context length");
    rows += (n + max_block - 1) / max_block;
  }
  *num_rows = rows;
  if (!row_seq) return PA_OK;  // size query
  if (!row_lens || !row_qsl || capacity < rows)
    return pa::fail(PA_EINVAL, "pa_query_blocks: outputs missing or capacity too small");
  int64_t r = 0;
  row_qsl[0] = query_start_loc[0];
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t q0 = query_start_loc[s];
    const int32_t n = query_start_loc[s + 1] - q0;
    const int32_t first = context_lens[s] - n;  // position of the first new token
    for (int32_t j = 0; j < n; j += max_block) {
      const int32_t e = std::min(n, j + max_block);
      row_seq[r] = s;
      row_lens[r] = first + e;
      row_qsl[r + 1] = q0 + e;
      ++r;
    }
  }
  return PA_OK;
}

// A sequence cut into several rows has every block of its context read by
// each of them, so all of a row's blocks are shared then; a sequence with one
// row keeps its own shared prefix.
extern "C" int32_t pa_query_block_hints(const int32_t* row_seq, const int32_t* row_lens,
                                        int32_t num_rows, const int32_t* seq_shared_blocks,
                                        int32_t num_seqs, int32_t block_size,
                                        int32_t* row_shared_out) {
  if (!row_seq || !row_lens || !row_shared_out || num_rows < 1 || num_seqs < 1 ||
      block_size < 1)
    return pa::fail(PA_EINVAL, "pa_query_block_hints: bad argument");
  std::vector<int32_t> rows_of(num_seqs, 0);
  for (int32_t r = 0; r < num_rows; ++r) {
    if (row_seq[r] < 0 || row_seq[r] >= num_seqs || row_lens[r] < 0)
      return pa::fail(PA_EINVAL, "pa_query_block_hints: row sequence or length out of range");
    ++rows_of[row_seq[r]];
  }
  for (int32_t r = 0; r < num_rows; ++r) {
    const int32_t s = row_seq[r];
    row_shared_out[r] = rows_of[s] > 1
                            ? static_cast<int32_t>((static_cast<int64_t>(row_lens[r]) +
                                                    block_size - 1) / block_size)
                            : (seq_shared_blocks ? seq_shared_blocks[s] : 0);
  }
  return PA_OK;
}

// Launch order of the prefill kernel's rows: sequences by their largest
// row (keys read), largest first, a sequence's rows together, largest first.
extern "C" int32_t pa_prefill_plan(const int32_t* row_seq, const int32_t* row_lens,
                                   const int32_t* row_qlens, int32_t num_rows,
                                   int32_t sliding_window, int32_t* items) {
  if (!row_seq || !row_lens || !items || num_rows < 1 || sliding_window < 0)
    return pa::fail(PA_EINVAL, "pa_prefill_plan: bad argument");
  std::vector<int64_t> size(num_rows);
  std::map<int32_t, int64_t> seq_size;
  for (int32_t r = 0; r < num_rows; ++r) {
    const int64_t L = row_lens[r];
    const int64_t n = row_qlens ? row_qlens[r] : 1;
    if (row_seq[r] < 0 || L < 0 || n < 0 || n > L)
      return pa::fail(PA_EINVAL, "pa_prefill_plan: row sequence, length or tokens out of range");
    const int64_t lo = sliding_window > 0 ? std::max<int64_t>(0, L - n + 1 - sliding_window) : 0;
    size[r] = L - lo;
    int64_t& m = seq_size[row_seq[r]];
    m = std::max(m, size[r]);
  }
  std::vector<int64_t> seq_key(num_rows);
  std::vector<int32_t> order(num_rows);
  for (int32_t r = 0; r < num_rows; ++r) {
    seq_key[r] = seq_size[row_seq[r]];
    order[r] = r;
  }
  std::sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
    if (seq_key[a] != seq_key[b]) return seq_key[a] > seq_key[b];
    if (row_seq[a] != row_seq[b]) return row_seq[a] < row_seq[b];
    if (size[a] != size[b]) return size[a] > size[b];
    return a < b;
  });
  for (int32_t i = 0; i < num_rows; ++i) {
    items[2 * i] = order[i];
    items[2 * i + 1] = 0;
  }
  return PA_OK;
}

// Split launch order of the prefill kernel: per row, the partitions from the
// one holding its first visible key to the one holding its last; sequences
// by their largest row, largest first, and within a sequence by partition,
// then by row size, so that the items reading one partition's rows run
// together.
extern "C" int32_t pa_prefill_plan_split(const int32_t* row_seq, const int32_t* row_lens,
                                         const int32_t* row_qlens, int32_t num_rows,
                                         int32_t sliding_window, int32_t partition_size,
                                         int32_t* items, int64_t capacity, int64_t* num_items) {
  if (!row_seq || !row_lens || !num_items || num_rows < 1 || sliding_window < 0 ||
      partition_size < 1)
    return pa::fail(PA_EINVAL, "pa_prefill_plan_split: bad argument");
  struct Item {
    int32_t row, part;
  };
  std::vector<Item> all;
  std::vector<int64_t> size(num_rows);
  std::map<int32_t, int64_t> seq_size;
  for (int32_t r = 0; r < num_rows; ++r) {
    const int64_t L = row_lens[r];
    const int64_t n = row_qlens ? row_qlens[r] : 1;
    if (row_seq[r] < 0 || L < 1 || n < 0 || n > L)
      return pa::fail(PA_EINVAL,
                      "pa_prefill_plan_split: row sequence, length or tokens out of range");
    const int64_t lo = sliding_window > 0 ? std::max<int64_t>(0, L - n + 1 - sliding_window) : 0;
    size[r] = L - lo;
    int64_t& m = seq_size[row_seq[r]];
    m = std::max(m, size[r]);
    const int64_t p_end = (L + partition_size - 1) / partition_size;
    for (int64_t p = lo / partition_size; p < p_end; ++p)
      all.push_back({r, static_cast<int32_t>(p)});
  }
  *num_items = static_cast<int64_t>(all.size());
  if (!items) return PA_OK;
  if (capacity < *num_items)
    return pa::fail(PA_EINVAL, "pa_prefill_plan_split: capacity below the item count");
  std::sort(all.begin(), all.end(), [&](const Item& a, const Item& b) {
    const int64_t sa = seq_size[row_seq[a.row]], sb = seq_size[row_seq[b.row]];
    if (sa != sb) return sa > sb;
    if (row_seq[a.row] != row_seq[b.row]) return row_seq[a.row] < row_seq[b.row];
    if (a.part != b.part) return a.part < b.part;
    if (size[a.row] != size[b.row]) return size[a.row] > size[b.row];
    return a.row < b.row;
  });
  for (size_t i = 0; i < all.size(); ++i) {
    items[2 * i] = all[i].row;
    items[2 * i + 1] = all[i].part;
  }
  return PA_OK;
}

// Partitions for the split prefill when one pass leaves the GPU mostly idle:
// fewer (row, KV head) workgroups than two per CU of an MI355X (256 CUs) and
// a row of at least 8192 keys; 0 otherwise.
extern "C" int32_t pa_prefill_auto_partition(int32_t num_rows, int32_t num_kv_heads,
                                             int32_t max_row_len, int32_t block_size,
                                             int32_t* partition_size) {
  if (!partition_size || num_rows < 1 || num_kv_heads < 1 || max_row_len < 0 || block_size < 1)
    return pa::fail(PA_EINVAL, "pa_prefill_auto_partition: bad argument");
  constexpr int64_t kSlots = 2 * 256;
  constexpr int32_t kPartition = 4096;
  const bool few = static_cast<int64_t>(num_rows) * num_kv_heads < kSlots;
  *partition_size =
      few && max_row_len >= 2 * kPartition && kPartition % block_size == 0 ? kPartition : 0;
  return PA_OK;
}

// Members whose decode queries fill the matrix cores' 16 columns of a group
// item: 16 / (num_heads / num_kv_heads), at most 8; 0 where the group items'
// kernels do not exist (fp32 storage, head_size other than 128).
extern "C" int32_t pa_cascade_max_group(int32_t num_heads, int32_t num_kv_heads,
                                        int32_t head_size, int32_t dtype, int32_t* group) {
  if (!group || num_heads < 1 || num_kv_heads < 1 || num_heads % num_kv_heads != 0)
    return pa::fail(PA_EINVAL, "pa_cascade_max_group: bad arguments");
  const int32_t g = num_heads / num_kv_heads;
  *group = ((dtype == PA_F16 || dtype == PA_BF16) && head_size == 128 && g <= 16)
               ? std::min(8, 16 / g)
               : 0;
  return PA_OK;
}
