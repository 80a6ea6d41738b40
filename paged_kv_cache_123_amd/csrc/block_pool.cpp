// Host block allocator: physical block pool with reference counts and
// copy-on-write, producing the block tables and slots the kernels consume,
// with an optional prefix cache over its blocks ([DEEPSONAR] section 2.4;
// [CSDN] sections 3.2.1-3.2.3 and 5.2-5.3): full blocks are keyed by a
// chained SHA-256, a new request takes over its longest cached prefix, and
// the free queue is the LRU list whose head is evicted when reused.
//
// Semantics ([PUFANYI] "按 Block 分配"; [CSDN] sections 3.1.2, 3.2.1, 3.2.3,
// 3.2.4; [VLLBC] paper section 4.4 / Fig. 8) are described in pagedkv.h.
// With a sliding window, the blocks a sequence's next query can no longer see
// are released early ([CSDN] sections 3.1.1 and 3.3.1); they leave holes (-1)
// at the front of its table.
// Design: the free queue is an intrusive doubly linked list over block ids
// (prev/next arrays), so taking the head, appending at the tail and removing
// an arbitrary block are all O(1) with no allocation after creation.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <string>
#include <unordered_map>
#include <vector>

#include "pagedkv.h"
#include "sha256.h"
#include "status.h"

namespace {

struct Seq {
  std::vector<int32_t> blocks;
  int64_t len = 0;
  // prefix caching: the token ids behind the blocks (tracked == false once
  // tokens were appended without ids) and the request's extra key bytes
  bool tracked = false;
  std::vector<int32_t> tokens;
  std::string extra;
  std::vector<pa::Digest> keys;  // keys of the first keys.size() full blocks
  size_t registered = 0;         // full blocks already offered to the cache
};

struct DigestHash {
  size_t operator()(const pa::Digest& d) const {
    size_t h;
    std::memcpy(&h, d.data(), sizeof h);
    return h;
  }
};

// Key of one full block: SHA-256 of parent key || int32 LE token ids || extra.
pa::Digest block_key(const pa::Digest& parent, const int32_t* tokens, int32_t n,
                     const std::string& extra) {
  std::vector<uint8_t> tok(static_cast<size_t>(n) * 4);
  for (int32_t i = 0; i < n; ++i) {
    const uint32_t v = static_cast<uint32_t>(tokens[i]);
    for (int b = 0; b < 4; ++b) tok[4 * i + b] = static_cast<uint8_t>(v >> (8 * b));
  }
  const uint8_t* parts[3] = {parent.data(), tok.data(),
                             reinterpret_cast<const uint8_t*>(extra.data())};
  const size_t sizes[3] = {parent.size(), tok.size(), extra.size()};
  return pa::sha256(parts, sizes, 3);
}

// Extend a chain of block keys to the full blocks of tokens[0, n): each key
// chains on the one before, the first block's parent being 32 zero bytes.
void extend_keys(std::vector<pa::Digest>& keys, const int32_t* tokens, int64_t n,
                 int32_t block_size, const std::string& extra) {
  for (int64_t j = static_cast<int64_t>(keys.size()); (j + 1) * block_size <= n; ++j) {
    const pa::Digest parent = j > 0 ? keys[j - 1] : pa::Digest{};
    keys.push_back(block_key(parent, tokens + j * block_size, block_size, extra));
  }
}

}  // namespace

struct pa_pool {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> ref;
  // Free queue as a linked list; kNone marks list ends / "not queued".
  static constexpr int32_t kNone = -1;
  std::vector<int32_t> prev, next;
  std::vector<uint8_t> queued;
  int32_t head = kNone, tail = kNone, num_free = 0;
  std::unordered_map<int64_t, Seq> seqs;
  int64_t num_cow = 0;
  // prefix cache: key of each cached block, and key -> block
  bool caching = false;
  std::vector<pa::Digest> key_of;
  std::vector<uint8_t> has_key;
  std::unordered_map<pa::Digest, int32_t, DigestHash> cached;
  int64_t num_evicted = 0;

  void push_tail(int32_t b) {
    prev[b] = tail;
    next[b] = kNone;
    if (tail != kNone) next[tail] = b; else head = b;
    tail = b;
    queued[b] = 1;
    ++num_free;
  }
  int32_t pop_head() {
    int32_t b = head;
    head = next[b];
    if (head != kNone) prev[head] = kNone; else tail = kNone;
    prev[b] = next[b] = kNone;
    queued[b] = 0;
    --num_free;
    return b;
  }
  void unlink(int32_t b) {  // take b out of the free queue wherever it is
    if (prev[b] != kNone) next[prev[b]] = next[b]; else head = next[b];
    if (next[b] != kNone) prev[next[b]] = prev[b]; else tail = prev[b];
    prev[b] = next[b] = kNone;
    queued[b] = 0;
    --num_free;
  }
  int32_t take() {  // caller checked num_free
    int32_t b = pop_head();
    if (caching && has_key[b]) {  // the LRU head still holds cached content
      auto it = cached.find(key_of[b]);
      if (it != cached.end() && it->second == b) cached.erase(it);
      has_key[b] = 0;
      ++num_evicted;
    }
    ref[b] = 1;
    return b;
  }
  void touch(int32_t b) {  // a cache hit: a block without holders leaves the queue
    if (ref[b] == 0) unlink(b);
    ref[b] += 1;
  }
  int64_t fresh_blocks_needed(const Seq& s, int32_t n) const {
    const int64_t B = block_size;
    int64_t need = 0;
    if (s.len % B != 0 && ref[s.blocks.back()] > 1) need += 1;  // copy of the shared tail
    need += (s.len + n + B - 1) / B - (s.len + B - 1) / B;
    return need;
  }
};

extern "C" {

int32_t pa_pool_create(int32_t num_blocks, int32_t block_size,
                       const int32_t* initial_free_order, pa_pool** out) {
  if (!out) return pa::fail(PA_EINVAL, "pa_pool_create: out is NULL");
  *out = nullptr;
  if (num_blocks < 1 || block_size < 1)
    return pa::fail(PA_EINVAL, "pa_pool_create: num_blocks and block_size must be >= 1");
  auto* p = new pa_pool();
  p->num_blocks = num_blocks;
  p->block_size = block_size;
  p->ref.assign(num_blocks, 0);
  p->prev.assign(num_blocks, pa_pool::kNone);
  p->next.assign(num_blocks, pa_pool::kNone);
  p->queued.assign(num_blocks, 0);
  for (int32_t i = 0; i < num_blocks; ++i) {
    int32_t b = initial_free_order ? initial_free_order[i] : i;
    if (b < 0 || b >= num_blocks || p->queued[b]) {
      delete p;
      return pa::fail(PA_EINVAL, "pa_pool_create: initial_free_order is not a permutation");
    }
    p->push_tail(b);
  }
  *out = p;
  return PA_OK;
}

void pa_pool_destroy(pa_pool* pool) { delete pool; }

int32_t pa_pool_add_seq(pa_pool* pool, int64_t seq) {
  if (!pool) return pa::fail(PA_EINVAL, "pa_pool_add_seq: pool is NULL");
  if (pool->seqs.count(seq)) return pa::fail(PA_EINVAL, "pa_pool_add_seq: sequence exists");
  pool->seqs.emplace(seq, Seq{});
  return PA_OK;
}

int32_t pa_pool_fork(pa_pool* pool, int64_t parent, int64_t child) {
  if (!pool) return pa::fail(PA_EINVAL, "pa_pool_fork: pool is NULL");
  auto it = pool->seqs.find(parent);
  if (it == pool->seqs.end()) return pa::fail(PA_EINVAL, "pa_pool_fork: unknown parent");
  if (pool->seqs.count(child)) return pa::fail(PA_EINVAL, "pa_pool_fork: child exists");
  Seq c = it->second;
  for (int32_t b : c.blocks)
    if (b >= 0) pool->ref[b] += 1;
  pool->seqs.emplace(child, std::move(c));
  return PA_OK;
}

int32_t pa_pool_append(pa_pool* pool, int64_t seq, int32_t n, int64_t* slots_out,
                       int64_t* cow_pair_out, int32_t* n_cow_out) {
  if (!pool || !slots_out) return pa::fail(PA_EINVAL, "pa_pool_append: NULL argument");
  if (n < 1) return pa::fail(PA_EINVAL, "pa_pool_append: n must be >= 1");
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end()) return pa::fail(PA_EINVAL, "pa_pool_append: unknown sequence");
  Seq& s = it->second;
  const int64_t B = pool->block_size;
  const bool will_copy = s.len % B != 0 && pool->ref[s.blocks.back()] > 1;
  if (will_copy && !cow_pair_out)
    return pa::fail(PA_EINVAL, "pa_pool_append: a copy is needed but cow_pair_out is NULL");
  if (pool->fresh_blocks_needed(s, n) > pool->num_free)
    return pa::fail(PA_ENOMEM, "pa_pool_append: not enough free blocks");
  if (n_cow_out) *n_cow_out = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (s.len % B == 0) {
      s.blocks.push_back(pool->take());
    } else if (pool->ref[s.blocks.back()] > 1) {
      const int32_t old = s.blocks.back();
      const int32_t fresh = pool->take();
      pool->ref[old] -= 1;
      s.blocks.back() = fresh;
      cow_pair_out[0] = old;
      cow_pair_out[1] = fresh;
      if (n_cow_out) *n_cow_out = 1;
      pool->num_cow += 1;
    }
    slots_out[i] = static_cast<int64_t>(s.blocks[s.len / B]) * B + s.len % B;
    s.len += 1;
  }
  s.tracked = false;  // token ids unknown from here on: no longer cacheable
  return PA_OK;
}

int32_t pa_pool_free_seq(pa_pool* pool, int64_t seq) {
  if (!pool) return pa::fail(PA_EINVAL, "pa_pool_free_seq: pool is NULL");
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end()) return pa::fail(PA_EINVAL, "pa_pool_free_seq: unknown sequence");
  const std::vector<int32_t>& blocks = it->second.blocks;
  for (auto b = blocks.rbegin(); b != blocks.rend(); ++b) {
    if (*b >= 0 && --pool->ref[*b] == 0) pool->push_tail(*b);
  }
  pool->seqs.erase(it);
  return PA_OK;
}

int32_t pa_pool_remove_skipped(pa_pool* pool, int64_t seq, int64_t num_computed_tokens,
                               int32_t sliding_window, int32_t* num_released) {
  if (!pool || num_computed_tokens < 0 || sliding_window < 0)
    return pa::fail(PA_EINVAL, "pa_pool_remove_skipped: bad argument");
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end())
    return pa::fail(PA_EINVAL, "pa_pool_remove_skipped: unknown sequence");
  std::vector<int32_t>& blocks = it->second.blocks;
  // the next query (position num_computed_tokens) sees the last W positions
  const int64_t skipped =
      sliding_window > 0 ? std::max<int64_t>(0, num_computed_tokens - sliding_window + 1) : 0;
  const int64_t n = std::min<int64_t>(skipped / pool->block_size,
                                      static_cast<int64_t>(blocks.size()));
  int32_t released = 0;
  for (int64_t j = n - 1; j >= 0; --j) {  // tail first, as a freed request
    const int32_t b = blocks[j];
    if (b < 0) continue;
    blocks[j] = -1;
    if (--pool->ref[b] == 0) pool->push_tail(b);
    ++released;
  }
  if (num_released) *num_released = released;
  return PA_OK;
}

int32_t pa_pool_append_batch(pa_pool* pool, const int64_t* seqs, const int32_t* num_new,
                             int32_t num_seqs, int32_t sliding_window,
                             int32_t blocks_per_kv_block, int64_t* positions_out,
                             int32_t* query_start_loc_out, int64_t* slots_out,
                             int64_t* cow_src_out, int64_t* cow_pairs_out,
                             int32_t* num_cow_pairs_out, int32_t* shared_blocks_out,
                             int32_t* group_keys_out) {
  if (!pool || !seqs || !num_new || !positions_out || !query_start_loc_out || !cow_src_out ||
      !cow_pairs_out || !num_cow_pairs_out)
    return pa::fail(PA_EINVAL, "pa_pool_append_batch: NULL argument");
  if (num_seqs < 1 || sliding_window < 0 || blocks_per_kv_block < 1)
    return pa::fail(PA_EINVAL, "pa_pool_append_batch: bad num_seqs, sliding_window or "
                               "blocks_per_kv_block");
  const int64_t k = blocks_per_kv_block;
  if (static_cast<int64_t>(pool->num_blocks) * k > INT32_MAX)
    return pa::fail(PA_EINVAL, "pa_pool_append_batch: kernel block ids overflow int32");
  // Dry run: every row is checked and the free queue is followed row by row
  // (window releases first, then the copy of a shared tail and the fresh
  // blocks) on an overlay of the reference counts, so that a step either
  // fits as a whole or leaves the pool untouched.
  std::unordered_map<int64_t, int32_t> row_of;
  std::unordered_map<int32_t, int32_t> ref_now;  // counts the dry run changed
  auto ref_of = [&](int32_t b) {
    auto it = ref_now.find(b);
    return it != ref_now.end() ? it->second : pool->ref[b];
  };
  const int64_t B = pool->block_size;
  int64_t free_now = pool->num_free, total = 0;
  for (int32_t r = 0; r < num_seqs; ++r) {
    auto it = pool->seqs.find(seqs[r]);
    if (it == pool->seqs.end())
      return pa::fail(PA_EINVAL, "pa_pool_append_batch: unknown sequence");
    if (!row_of.emplace(seqs[r], r).second)
      return pa::fail(PA_EINVAL, "pa_pool_append_batch: a sequence is listed twice");
    if (num_new[r] < 1)
      return pa::fail(PA_EINVAL, "pa_pool_append_batch: every row appends at least one token");
    total += num_new[r];
    if (total > INT32_MAX) return pa::fail(PA_EINVAL, "pa_pool_append_batch: too many tokens");
    const Seq& s = it->second;
    if (sliding_window > 0) {
      const int64_t skipped = std::max<int64_t>(0, s.len - sliding_window + 1);
      const int64_t n = std::min<int64_t>(skipped / B, static_cast<int64_t>(s.blocks.size()));
      for (int64_t j = n - 1; j >= 0; --j) {
        const int32_t b = s.blocks[j];
        if (b < 0) continue;
        const int32_t c = ref_of(b) - 1;
        ref_now[b] = c;
        if (c == 0) ++free_now;
      }
    }
    if (s.len % B != 0) {
      const int32_t tail = s.blocks.back();
      if (ref_of(tail) > 1) {  // copy-on-write: one fresh block, one holder less
        ref_now[tail] = ref_of(tail) - 1;
        --free_now;
      }
    }
    free_now -= (s.len + num_new[r] + B - 1) / B - (s.len + B - 1) / B;
    if (free_now < 0) return pa::fail(PA_ENOMEM, "pa_pool_append_batch: not enough free blocks");
  }
  // The step itself: each row releases, then appends (cannot fail now).
  int64_t t = 0;
  int32_t pairs = 0;
  query_start_loc_out[0] = 0;
  for (int32_t r = 0; r < num_seqs; ++r) {
    const int64_t start = pool->seqs.find(seqs[r])->second.len;
    if (sliding_window > 0) pa_pool_remove_skipped(pool, seqs[r], start, sliding_window, nullptr);
    int64_t pair[2];
    int32_t copied = 0;
    std::vector<int64_t> row_slots;
    int64_t* sl = slots_out ? slots_out + t : (row_slots.resize(num_new[r]), row_slots.data());
    const int32_t st = pa_pool_append(pool, seqs[r], num_new[r], sl, pair, &copied);
    if (st != PA_OK) return st;  // unreachable after the dry run
    for (int32_t i = 0; i < num_new[r]; ++i) positions_out[t + i] = start + i;
    t += num_new[r];
    query_start_loc_out[r + 1] = static_cast<int32_t>(t);
    cow_src_out[r] = copied ? pair[0] : -1;
    if (copied) {
      for (int64_t j = 0; j < k; ++j) {
        cow_pairs_out[2 * pairs] = pair[0] * k + j;
        cow_pairs_out[2 * pairs + 1] = pair[1] * k + j;
        ++pairs;
      }
    }
  }
  *num_cow_pairs_out = pairs;
  if (shared_blocks_out || group_keys_out) {
    std::vector<int32_t> shared(num_seqs);
    pa_pool_shared_prefix_blocks(pool, seqs, num_seqs, shared.data());
    for (int32_t r = 0; r < num_seqs; ++r) {
      if (shared_blocks_out) shared_blocks_out[r] = static_cast<int32_t>(shared[r] * k);
      if (!group_keys_out) continue;
      // readers of one shared prefix share a key: its first live block, in
      // kernel blocks; a row without shared blocks gets a key of its own
      int32_t key = static_cast<int32_t>(pool->num_blocks * k + r);
      if (shared[r] > 0) {
        for (int32_t b : pool->seqs.find(seqs[r])->second.blocks) {
          if (b >= 0) {
            key = static_cast<int32_t>(b * k);
            break;
          }
        }
      }
      group_keys_out[r] = key;
    }
  }
  return PA_OK;
}

int32_t pa_pool_seq_len(const pa_pool* pool, int64_t seq, int64_t* len_out) {
  if (!pool || !len_out) return pa::fail(PA_EINVAL, "pa_pool_seq_len: NULL argument");
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end()) return pa::fail(PA_EINVAL, "pa_pool_seq_len: unknown sequence");
  *len_out = it->second.len;
  return PA_OK;
}

int32_t pa_pool_seq_num_blocks(const pa_pool* pool, int64_t seq, int32_t* n_out) {
  if (!pool || !n_out) return pa::fail(PA_EINVAL, "pa_pool_seq_num_blocks: NULL argument");
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end())
    return pa::fail(PA_EINVAL, "pa_pool_seq_num_blocks: unknown sequence");
  *n_out = static_cast<int32_t>(it->second.blocks.size());
  return PA_OK;
}

int32_t pa_pool_block_tables(const pa_pool* pool, const int64_t* seqs, int32_t num_seqs,
                             int32_t* out, int32_t width, int32_t* context_lens_out) {
  if (!pool || !seqs || !out) return pa::fail(PA_EINVAL, "pa_pool_block_tables: NULL argument");
  if (num_seqs < 0 || width < 1)
    return pa::fail(PA_EINVAL, "pa_pool_block_tables: bad num_seqs or width");
  for (int32_t r = 0; r < num_seqs; ++r) {
    auto it = pool->seqs.find(seqs[r]);
    if (it == pool->seqs.end())
      return pa::fail(PA_EINVAL, "pa_pool_block_tables: unknown sequence");
    if (static_cast<int64_t>(it->second.blocks.size()) > width)
      return pa::fail(PA_EINVAL, "pa_pool_block_tables: table wider than width");
  }
  for (int32_t r = 0; r < num_seqs; ++r) {
    const Seq& s = pool->seqs.find(seqs[r])->second;
    int32_t* row = out + static_cast<int64_t>(r) * width;
    const int32_t nb = static_cast<int32_t>(s.blocks.size());
    for (int32_t j = 0; j < width; ++j) row[j] = j < nb ? s.blocks[j] : -1;
    if (context_lens_out) context_lens_out[r] = static_cast<int32_t>(s.len);
  }
  return PA_OK;
}

int32_t pa_pool_shared_prefix_blocks(const pa_pool* pool, const int64_t* seqs, int32_t num_seqs,
                                     int32_t* out) {
  if (!pool || !seqs || !out || num_seqs < 0)
    return pa::fail(PA_EINVAL, "pa_pool_shared_prefix_blocks: bad argument");
  for (int32_t r = 0; r < num_seqs; ++r) {
    auto it = pool->seqs.find(seqs[r]);
    if (it == pool->seqs.end())
      return pa::fail(PA_EINVAL, "pa_pool_shared_prefix_blocks: unknown sequence");
    // holes (released blocks) are never read: they may sit inside the prefix,
    // which ends after its last shared block
    int32_t n = 0, j = 0;
    for (int32_t b : it->second.blocks) {
      ++j;
      if (b < 0) continue;
      if (pool->ref[b] <= 1) break;
      n = j;
    }
    out[r] = n;
  }
  return PA_OK;
}

int32_t pa_pool_num_free(const pa_pool* pool) { return pool ? pool->num_free : -1; }

int32_t pa_pool_ref(const pa_pool* pool, int32_t block) {
  if (!pool || block < 0 || block >= pool->num_blocks) return -1;
  return pool->ref[block];
}

int32_t pa_pool_free_queue(const pa_pool* pool, int32_t* out, int32_t cap) {
  if (!pool || (!out && cap > 0)) return -1;
  int32_t n = 0;
  for (int32_t b = pool->head; b != pa_pool::kNone && n < cap; b = pool->next[b]) out[n++] = b;
  return n;
}

int64_t pa_pool_num_cow(const pa_pool* pool) { return pool ? pool->num_cow : -1; }

int32_t pa_pool_enable_prefix_caching(pa_pool* pool) {
  if (!pool) return pa::fail(PA_EINVAL, "pa_pool_enable_prefix_caching: pool is NULL");
  if (!pool->seqs.empty())
    return pa::fail(PA_EINVAL, "pa_pool_enable_prefix_caching: the pool already has sequences");
  pool->caching = true;
  pool->key_of.assign(pool->num_blocks, pa::Digest{});
  pool->has_key.assign(pool->num_blocks, 0);
  return PA_OK;
}

int32_t pa_pool_add_seq_cached(pa_pool* pool, int64_t seq, const int32_t* prompt,
                               int64_t num_prompt_tokens, const void* extra,
                               int32_t extra_bytes, int64_t* num_computed_tokens) {
  if (!pool || (!prompt && num_prompt_tokens > 0) || num_prompt_tokens < 0 || extra_bytes < 0 ||
      (!extra && extra_bytes > 0) || !num_computed_tokens)
    return pa::fail(PA_EINVAL, "pa_pool_add_seq_cached: bad argument");
  if (!pool->caching)
    return pa::fail(PA_EINVAL, "pa_pool_add_seq_cached: prefix caching is not enabled");
  if (pool->seqs.count(seq)) return pa::fail(PA_EINVAL, "pa_pool_add_seq_cached: sequence exists");
  Seq s;
  s.tracked = true;
  if (extra_bytes > 0) s.extra.assign(static_cast<const char*>(extra), extra_bytes);
  // the last prompt token is always computed again: at most n - 1 from the
  // cache; keys are hashed block by block up to the first miss
  const int64_t B = pool->block_size;
  const int64_t max_blocks = num_prompt_tokens > 0 ? (num_prompt_tokens - 1) / B : 0;
  for (int64_t j = 0; j < max_blocks; ++j) {
    extend_keys(s.keys, prompt, (j + 1) * B, pool->block_size, s.extra);
    auto it = pool->cached.find(s.keys[j]);
    if (it == pool->cached.end()) break;
    s.blocks.push_back(it->second);
  }
  s.registered = s.blocks.size();  // taken-over blocks are cached already
  for (int32_t b : s.blocks) pool->touch(b);
  s.len = static_cast<int64_t>(s.blocks.size()) * pool->block_size;
  s.tokens.assign(prompt, prompt + s.len);
  *num_computed_tokens = s.len;
  pool->seqs.emplace(seq, std::move(s));
  return PA_OK;
}

int32_t pa_pool_append_tokens(pa_pool* pool, int64_t seq, const int32_t* tokens, int32_t n,
                              int64_t* slots_out, int64_t* cow_pair_out, int32_t* n_cow_out) {
  if (!pool || !tokens) return pa::fail(PA_EINVAL, "pa_pool_append_tokens: NULL argument");
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end())
    return pa::fail(PA_EINVAL, "pa_pool_append_tokens: unknown sequence");
  const bool tracked = it->second.tracked;
  const int32_t st = pa_pool_append(pool, seq, n, slots_out, cow_pair_out, n_cow_out);
  if (st != PA_OK) return st;
  Seq& s = pool->seqs.find(seq)->second;
  s.tracked = tracked;
  if (tracked) s.tokens.insert(s.tokens.end(), tokens, tokens + n);
  return PA_OK;
}

int32_t pa_pool_cache_full_blocks(pa_pool* pool, int64_t seq, int32_t* num_cached) {
  if (!pool) return pa::fail(PA_EINVAL, "pa_pool_cache_full_blocks: pool is NULL");
  if (!pool->caching)
    return pa::fail(PA_EINVAL, "pa_pool_cache_full_blocks: prefix caching is not enabled");
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end())
    return pa::fail(PA_EINVAL, "pa_pool_cache_full_blocks: unknown sequence");
  Seq& s = it->second;
  if (!s.tracked)
    return pa::fail(PA_EINVAL, "pa_pool_cache_full_blocks: the sequence's token ids are unknown");
  extend_keys(s.keys, s.tokens.data(), s.len, pool->block_size, s.extra);
  const size_t full = static_cast<size_t>(s.len / pool->block_size);
  int32_t n = 0;
  for (size_t j = s.registered; j < full; ++j) {
    const int32_t b = s.blocks[j];
    if (b < 0 || pool->has_key[b]) continue;
    if (pool->cached.count(s.keys[j])) continue;  // another block holds this content
    pool->key_of[b] = s.keys[j];
    pool->has_key[b] = 1;
    pool->cached.emplace(s.keys[j], b);
    ++n;
  }
  s.registered = std::max(s.registered, full);
  if (num_cached) *num_cached = n;
  return PA_OK;
}

int64_t pa_pool_num_cached_blocks(const pa_pool* pool) {
  return pool ? static_cast<int64_t>(pool->cached.size()) : -1;
}

int64_t pa_pool_num_evicted(const pa_pool* pool) { return pool ? pool->num_evicted : -1; }

int32_t pa_block_keys(const int32_t* tokens, int64_t num_tokens, int32_t block_size,
                      const void* extra, int32_t extra_bytes, uint8_t* keys_out) {
  if ((!tokens && num_tokens > 0) || num_tokens < 0 || block_size < 1 || extra_bytes < 0 ||
      (!extra && extra_bytes > 0) || (!keys_out && num_tokens >= block_size))
    return pa::fail(PA_EINVAL, "pa_block_keys: bad argument");
  std::string x;
  if (extra_bytes > 0) x.assign(static_cast<const char*>(extra), extra_bytes);
  std::vector<pa::Digest> keys;
  extend_keys(keys, tokens, num_tokens, block_size, x);
  for (size_t j = 0; j < keys.size(); ++j) std::memcpy(keys_out + 32 * j, keys[j].data(), 32);
  return PA_OK;
}

int32_t pa_map_to_kernel_blocks(const int32_t* manager_ids, int64_t n,
                                int32_t blocks_per_kv_block, int32_t* kernel_ids) {
  if ((n > 0 && (!manager_ids || !kernel_ids)) || n < 0 || blocks_per_kv_block < 1)
    return pa::fail(PA_EINVAL, "pa_map_to_kernel_blocks: bad argument");
  const int64_t k = blocks_per_kv_block;
  for (int64_t i = 0; i < n; ++i)
    if (manager_ids[i] > (static_cast<int64_t>(INT32_MAX) - k + 1) / k)
      return pa::fail(PA_EINVAL, "pa_map_to_kernel_blocks: kernel block id overflows int32");
  for (int64_t i = 0; i < n; ++i) {
    const int64_t b = manager_ids[i];
    for (int64_t j = 0; j < k; ++j)
      kernel_ids[i * k + j] = b < 0 ? -1 : static_cast<int32_t>(b * k + j);
  }
  return PA_OK;
}

}  // extern "C"
