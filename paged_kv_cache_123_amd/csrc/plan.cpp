// Host-side work plan for the attention calls: every non-empty (sequence,
// partition) pair once, largest first, so that workgroups of a launch start
// in decreasing order of work and none is launched without work.  Sizes are
// compared in buckets of kGranule tokens and equal buckets keep batch order,
// so sequences that share blocks (forks of one prompt sit next to each other
// in a batch) still run close together in time and reuse cached blocks.
#include <algorithm>
#include <cstdint>
#include <vector>

#include "pagedkv.h"
#include "status.h"

namespace {
constexpr int32_t kGranule = 256;
}

extern "C" int32_t pa_decode_plan(const int32_t* context_lens, int32_t num_seqs,
                                  int32_t partition_size, int32_t* items, int64_t capacity,
                                  int64_t* num_items) {
  if (!context_lens || !num_items || num_seqs < 1 || partition_size < 0)
    return pa::fail(PA_EINVAL, "pa_decode_plan: bad argument");
  struct Item {
    int32_t tokens, s, p;
  };
  std::vector<Item> v;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t L = context_lens[s];
    if (L < 0 || (L == 0 && partition_size == 0))
      return pa::fail(PA_EINVAL, "pa_decode_plan: context length < 1");
    if (partition_size == 0) {
      v.push_back({L, s, 0});
      continue;
    }
    // a sequence with no token (a rank-local share can be empty) has no item
    for (int32_t p = 0; static_cast<int64_t>(p) * partition_size < L; ++p)
      v.push_back({std::min(partition_size, L - p * partition_size), s, p});
  }
  *num_items = static_cast<int64_t>(v.size());
  if (!items) return PA_OK;  // size query
  if (capacity < static_cast<int64_t>(v.size()))
    return pa::fail(PA_EINVAL, "pa_decode_plan: capacity smaller than the number of items");
  std::stable_sort(v.begin(), v.end(), [](const Item& a, const Item& b) {
    return (a.tokens + kGranule - 1) / kGranule > (b.tokens + kGranule - 1) / kGranule;
  });
  for (size_t i = 0; i < v.size(); ++i) {
    items[2 * i] = v[i].s;
    items[2 * i + 1] = v[i].p;
  }
  return PA_OK;
}
