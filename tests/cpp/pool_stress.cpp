// Host-only stress driver for the block pool and the work planner through the
// C ABI; built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitizers.py.  Exit status 0 = every check held.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "pagedkv.h"

#define CHECK(c)                                                     \
  do {                                                               \
    if (!(c)) {                                                      \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      return 1;                                                      \
    }                                                                \
  } while (0)

int main() {
  std::mt19937 rng(1234);
  for (int trial = 0; trial < 40; ++trial) {
    const int32_t B = 1 << (rng() % 7);
    const int32_t nb = 4 + static_cast<int32_t>(rng() % 200);
    std::vector<int32_t> order(nb);
    for (int32_t i = 0; i < nb; ++i) order[i] = i;
    std::shuffle(order.begin(), order.end(), rng);
    pa_pool* pool = nullptr;
    CHECK(pa_pool_create(nb, B, order.data(), &pool) == PA_OK);
    // odd trials: prefix caching, token-tracked sequences and sliding windows
    const bool caching = trial % 2 == 1;
    if (caching) CHECK(pa_pool_enable_prefix_caching(pool) == PA_OK);
    std::vector<int32_t> system(3 * B);
    for (auto& t : system) t = static_cast<int32_t>(rng() % 5);
    std::vector<int64_t> live;
    int64_t next = 0;
    for (int step = 0; step < 2000; ++step) {
      const unsigned op = rng() % 100;
      if (caching && op < 10) {  // a request over the shared system prompt
        std::vector<int32_t> prompt(system.begin(), system.begin() + rng() % (system.size() + 1));
        for (int i = 1 + static_cast<int>(rng() % (2 * B)); i > 0; --i)
          prompt.push_back(static_cast<int32_t>(rng() % 5));
        int64_t done = -1;
        CHECK(pa_pool_add_seq_cached(pool, next, prompt.data(), int64_t(prompt.size()), "x",
                                     int32_t(rng() % 2), &done) == PA_OK);
        CHECK(done >= 0 && done % B == 0 && done < int64_t(prompt.size()));
        const int32_t rest = static_cast<int32_t>(prompt.size() - done);
        std::vector<int64_t> slots(rest);
        int64_t pair[2];
        int32_t ncow = 0;
        const int32_t st = pa_pool_append_tokens(pool, next, prompt.data() + done, rest,
                                                 slots.data(), pair, &ncow);
        CHECK(st == PA_OK || st == PA_ENOMEM);
        int32_t ncached = -1;
        if (st == PA_OK) CHECK(pa_pool_cache_full_blocks(pool, next, &ncached) == PA_OK);
        live.push_back(next++);
        continue;
      }
      if (caching && op < 15) {  // a sliding window releases blocks behind it
        const int64_t s = live.empty() ? -1 : live[rng() % live.size()];
        if (s < 0) continue;
        int64_t len = 0;
        CHECK(pa_pool_seq_len(pool, s, &len) == PA_OK);
        int32_t nrel = -1;
        CHECK(pa_pool_remove_skipped(pool, s, len, 1 + static_cast<int32_t>(rng() % (4 * B)),
                                     &nrel) == PA_OK && nrel >= 0);
        continue;
      }
      if (op < 15 || live.empty()) {
        CHECK(pa_pool_add_seq(pool, next) == PA_OK);
        live.push_back(next++);
      } else if (op < 30) {
        const int64_t parent = live[rng() % live.size()];
        CHECK(pa_pool_fork(pool, parent, next) == PA_OK);
        live.push_back(next++);
      } else if (op < 42) {
        const size_t i = rng() % live.size();
        CHECK(pa_pool_free_seq(pool, live[i]) == PA_OK);
        live.erase(live.begin() + static_cast<std::ptrdiff_t>(i));
      } else {
        const int64_t s = live[rng() % live.size()];
        const int32_t n = 1 + static_cast<int32_t>(rng() % (3 * B));
        std::vector<int64_t> slots(n);
        int64_t pair[2] = {-1, -1};
        int32_t ncow = -1;
        int64_t len0 = 0;
        CHECK(pa_pool_seq_len(pool, s, &len0) == PA_OK);
        const int32_t st = pa_pool_append(pool, s, n, slots.data(), pair, &ncow);
        CHECK(st == PA_OK || st == PA_ENOMEM);
        if (st == PA_OK) {
          int64_t len1 = 0;
          CHECK(pa_pool_seq_len(pool, s, &len1) == PA_OK && len1 == len0 + n);
          for (int32_t i = 0; i < n; ++i) CHECK(slots[i] >= 0 && slots[i] < int64_t(nb) * B);
          CHECK(ncow == 0 || ncow == 1);
          if (ncow) CHECK(pair[0] != pair[1] && pa_pool_ref(pool, pair[1]) == 1);
        }
      }
      // invariants: reference counts equal table mappings; free <=> ref 0
      std::vector<int32_t> mapped(nb, 0);
      for (int64_t s : live) {
        int32_t k = 0;
        CHECK(pa_pool_seq_num_blocks(pool, s, &k) == PA_OK);
        std::vector<int32_t> row(k > 0 ? k : 1);
        int32_t len = 0;
        CHECK(pa_pool_block_tables(pool, &s, 1, row.data(), k > 0 ? k : 1, &len) == PA_OK);
        CHECK((len + B - 1) / B == k);
        for (int32_t j = 0; j < k; ++j)
          if (row[j] >= 0) mapped[row[j]] += 1;  // -1: released behind a window
        std::vector<int32_t> kern(2 * row.size());
        CHECK(pa_map_to_kernel_blocks(row.data(), int64_t(row.size()), 2, kern.data()) == PA_OK);
        for (size_t j = 0; j < row.size(); ++j)
          CHECK(kern[2 * j] == (row[j] < 0 ? -1 : 2 * row[j]));
      }
      if (caching) {
        CHECK(pa_pool_num_cached_blocks(pool) >= 0 && pa_pool_num_cached_blocks(pool) <= nb);
        CHECK(pa_pool_num_evicted(pool) >= 0);
      }
      std::vector<int32_t> q(nb);
      const int32_t nfree = pa_pool_free_queue(pool, q.data(), nb);
      CHECK(nfree == pa_pool_num_free(pool));
      std::vector<int> queued(nb, 0);
      for (int32_t i = 0; i < nfree; ++i) queued[q[i]] += 1;
      for (int32_t b = 0; b < nb; ++b) {
        CHECK(pa_pool_ref(pool, b) == mapped[b]);
        CHECK(queued[b] == (mapped[b] == 0 ? 1 : 0));
      }
    }
    pa_pool_destroy(pool);
  }
  // the planner: sizes, order and coverage
  for (int trial = 0; trial < 50; ++trial) {
    const int32_t S = 1 + static_cast<int32_t>(rng() % 300);
    const int32_t P = (rng() % 2) ? 0 : 16 * (1 + static_cast<int32_t>(rng() % 64));
    std::vector<int32_t> lens(S);
    for (auto& L : lens) L = 1 + static_cast<int32_t>(rng() % 9000);
    int64_t n = 0;
    CHECK(pa_decode_plan(lens.data(), S, P, nullptr, 0, &n) == PA_OK);
    std::vector<int32_t> items(2 * n);
    CHECK(pa_decode_plan(lens.data(), S, P, items.data(), n, &n) == PA_OK);
    int64_t want = 0;
    for (int32_t L : lens) want += P ? (L + P - 1) / P : 1;
    CHECK(n == want);
    for (int64_t i = 0; i < n; ++i) {
      const int32_t s = items[2 * i], p = items[2 * i + 1];
      CHECK(s >= 0 && s < S && p >= 0 && (P == 0 ? p == 0 : int64_t(p) * P < lens[s]));
    }
    if (n > 1) CHECK(pa_decode_plan(lens.data(), S, P, items.data(), n - 1, &n) == PA_EINVAL);
  }
  // windowed plans and context-parallel shares
  for (int trial = 0; trial < 50; ++trial) {
    const int32_t S = 1 + static_cast<int32_t>(rng() % 100);
    const int32_t P = 16 * (1 + static_cast<int32_t>(rng() % 8));
    const int32_t W = 1 + static_cast<int32_t>(rng() % 3000);
    std::vector<int32_t> lens(S), q(S), local(S);
    for (int32_t i = 0; i < S; ++i) {
      lens[i] = 1 + static_cast<int32_t>(rng() % 9000);
      q[i] = 1 + static_cast<int32_t>(rng() % std::min(lens[i], 8));
    }
    int64_t n = 0;
    CHECK(pa_decode_plan_window(lens.data(), q.data(), nullptr, S, P, W, nullptr, 0, &n) == PA_OK);
    std::vector<int32_t> items(2 * n + 2);
    CHECK(pa_decode_plan_window(lens.data(), q.data(), lens.data(), S, P, W, items.data(), n, &n) == PA_OK);
    const int32_t world = 1 + static_cast<int32_t>(rng() % 8);
    int64_t total = 0;
    for (int32_t r = 0; r < world; ++r) {
      CHECK(pa_cp_local_context_lens(lens.data(), S, 16, world, r, 1 << (rng() % 5),
                                     local.data()) == PA_OK);
      for (int32_t L : local) total += L;
    }
    (void)total;
  }
  std::puts("pool_stress ok");
  return 0;
}
