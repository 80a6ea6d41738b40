/* The C ABI used from plain C (C99): host-only calls, no GPU needed.
 * Exit status 0 = every check held. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "pagedkv.h"

#define CHECK(c)                                                        \
  do {                                                                  \
    if (!(c)) {                                                         \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);   \
      return 1;                                                         \
    }                                                                   \
  } while (0)

int main(void) {
  /* the 7-token growth example at B = 4, free order 7 1 3 4 5 0 2 6 */
  const int32_t order[8] = {7, 1, 3, 4, 5, 0, 2, 6};
  pa_pool* pool = NULL;
  CHECK(pa_pool_create(8, 4, order, &pool) == PA_OK);
  CHECK(pa_pool_add_seq(pool, 0) == PA_OK);
  int64_t slots[7], cow[2];
  int32_t ncow = -1;
  CHECK(pa_pool_append(pool, 0, 7, slots, cow, &ncow) == PA_OK && ncow == 0);
  CHECK(slots[0] == 28 && slots[3] == 31 && slots[4] == 4 && slots[6] == 6);
  CHECK(pa_pool_append(pool, 0, 1, slots, cow, &ncow) == PA_OK && slots[0] == 7);
  CHECK(pa_pool_append(pool, 0, 1, slots, cow, &ncow) == PA_OK && slots[0] == 12);
  int32_t table[4], len = 0;
  const int64_t seq = 0;
  CHECK(pa_pool_block_tables(pool, &seq, 1, table, 4, &len) == PA_OK);
  CHECK(len == 9 && table[0] == 7 && table[1] == 1 && table[2] == 3 && table[3] == -1);
  CHECK(pa_pool_append(pool, 9, 1, slots, cow, &ncow) == PA_EINVAL);
  CHECK(strlen(pa_last_error()) > 0);
  pa_pool_destroy(pool);

  /* planner, kernel blocks, context-parallel shares, block keys */
  const int32_t lens[3] = {40, 0, 17};
  int32_t items[16];
  int64_t n = 0;
  CHECK(pa_decode_plan(lens, 3, 16, items, 8, &n) == PA_OK && n == 5);
  const int32_t ids[2] = {0, 2};
  int32_t kids[4];
  CHECK(pa_map_to_kernel_blocks(ids, 2, 2, kids) == PA_OK);
  CHECK(kids[0] == 0 && kids[1] == 1 && kids[2] == 4 && kids[3] == 5);
  const int32_t clen[1] = {9};
  int32_t local[1];
  CHECK(pa_cp_local_context_lens(clen, 1, 4, 2, 1, 1, local) == PA_OK && local[0] == 4);
  const int32_t toks[4] = {1, 2, 3, 4};
  uint8_t key[32];
  CHECK(pa_block_keys(toks, 4, 4, NULL, 0, key) == PA_OK);
  CHECK(strcmp(pa_status_string(PA_ENOMEM), "") != 0);

  /* a prefill chunk cut into the prefill kernel's query blocks */
  const int32_t qlens[2] = {100, 30};
  const int32_t qsl[3] = {0, 70, 80};
  int32_t tokens = 0, rseq[8], rlen[8], rqsl[9];
  int64_t rows = 0;
  CHECK(pa_prefill_block_tokens(32, 8, &tokens) == PA_OK && tokens == 32);
  /* (blocks of 16 tokens here) */
  CHECK(pa_query_blocks(qlens, qsl, 2, 16, rseq, rlen, rqsl, 8, &rows) == PA_OK && rows == 6);
  CHECK(rlen[0] == 46 && rlen[4] == 100 && rseq[4] == 0 && rseq[5] == 1 && rlen[5] == 30);
  CHECK(rqsl[4] == 64 && rqsl[5] == 70 && rqsl[6] == 80);
  printf("abi_from_c ok %s\n", pa_version());
  return 0;
}
