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
#include <cstdint>
#include <vector>

#include "pagedkv.h"
#include "status.h"

namespace {
constexpr int32_t kGranule = 256;
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
