/* A C99 client of the library's C ABI: only include/pa.h and libpa.so, no
 * C++ and no Python.  Exercises the host-side block pool (no device calls)
 * and prints one line per check; exits non-zero on the first mismatch.
 * Built and run by tests/test_abi.py. */
#include <stdio.h>
#include <string.h>

#include "pa.h"

static int failures = 0;

#define CHECK(cond, what)                                   \
  do {                                                      \
    if (cond) {                                             \
      printf("ok   %s\n", what);                            \
    } else {                                                \
      printf("FAIL %s (line %d)\n", what, __LINE__);        \
      ++failures;                                           \
    }                                                       \
  } while (0)

int main(void) {
  /* free order: the first allocation returns 3, then 1, 4, 0, 5, 2, 7, 6 */
  const int32_t order[8] = {3, 1, 4, 0, 5, 2, 7, 6};
  const int32_t not_perm[4] = {0, 1, 1, 3};
  pa_pool* pool = NULL;
  pa_pool* bad = NULL;
  CHECK(pa_pool_create(4, not_perm, &bad) == PA_ERR_INVALID_ARG, "free order must be a permutation");
  CHECK(pa_pool_create(8, order, &pool) == PA_OK && pool != NULL, "pool of 8 blocks");

  /* sequence A: 20 tokens from position 0 take blocks 3 and 1 */
  int32_t row_a[8], nb_a = 0, src = 0, dst = 0;
  int64_t slots[20];
  CHECK(pa_append_slots(pool, row_a, &nb_a, 8, 0, 20, slots, &src, &dst) == PA_OK,
        "append 20 tokens");
  CHECK(nb_a == 2 && row_a[0] == 3 && row_a[1] == 1, "blocks taken in free order");
  CHECK(slots[0] == 3 * 16 && slots[15] == 3 * 16 + 15 && slots[16] == 1 * 16 &&
            slots[19] == 1 * 16 + 3,
        "slot = table[p / 16] * 16 + p % 16");
  CHECK(src == -1 && dst == -1, "no copy on a private append");

  /* sequence B shares A's blocks; its next token lands in shared block 1 */
  int32_t row_b[8], nb_b = 2;
  memcpy(row_b, row_a, sizeof(row_b));
  CHECK(pa_fork(pool, row_a, nb_a) == PA_OK, "fork");
  CHECK(pa_refcount(pool, 3) == 2 && pa_refcount(pool, 1) == 2, "shared blocks at count 2");
  int64_t slot_b = -1;
  CHECK(pa_append_slots(pool, row_b, &nb_b, 8, 20, 1, &slot_b, &src, &dst) == PA_OK,
        "append into a shared block");
  CHECK(src == 1 && dst == 4 && row_b[1] == 4, "copy on write: (1 -> 4), table repointed");
  CHECK(slot_b == 4 * 16 + 4, "the token goes to the copy");
  CHECK(pa_refcount(pool, 1) == 1 && pa_refcount(pool, 4) == 1 && pa_refcount(pool, 3) == 2,
        "counts after the copy");

  /* A finishes: block 3 stays (B holds it), block 1 returns and is reused first */
  CHECK(pa_free_table(pool, row_a, nb_a) == PA_OK, "free A");
  CHECK(pa_refcount(pool, 1) == 0 && pa_refcount(pool, 3) == 1, "counts after A");
  int32_t blk = -1;
  CHECK(pa_alloc(pool, &blk) == PA_OK && blk == 1, "a freed block is the next one out");
  CHECK(pa_free(pool, blk) == PA_OK, "free it again");
  CHECK(pa_free(pool, blk) == PA_ERR_BAD_BLOCK, "double free refused");
  CHECK(pa_incref(pool, 99) == PA_ERR_BAD_BLOCK, "id out of range refused");

  pa_pool_stats_t st;
  CHECK(pa_pool_stats(pool, &st) == PA_OK, "stats");
  CHECK(st.num_blocks == 8 && st.num_used == 2 && st.num_free == 6 && st.copies == 1,
        "stats: 2 held (3 and 4), 6 free, 1 copy");
  CHECK(pa_num_free(pool) == 6, "free count");

  /* drain the pool: 6 more allocations, then out of blocks with no change */
  int n = 0;
  while (pa_alloc(pool, &blk) == PA_OK) ++n;
  CHECK(n == 6 && pa_num_free(pool) == 0, "six allocations drain the pool");
  CHECK(pa_alloc(pool, &blk) == PA_ERR_OUT_OF_BLOCKS, "out of blocks");

  /* whole blocks for 10 GiB of a 70B-layer-shaped cache (80 layers, 8 KV
   * heads, head_dim 128, 2-byte elements): 327,680 bytes a token, 2048 blocks */
  CHECK(pa_blocks_for_bytes(10737418240LL, 80, 8, 128, 2) == 2048, "blocks for 10 GiB");

  pa_pool_destroy(pool);
  printf("%d failure(s)\n", failures);
  return failures == 0 ? 0 : 1;
}
