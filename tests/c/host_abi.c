/* A C99 program against include/pagedkv.h and libpagedkv.so that uses only
 * host entry points (no GPU): the block-table walk-through of "Why
 * PagedAttention multiplies LLM serving throughput" (section "Block Table:
 * the GPU page table"; also "vLLM PagedAttention explained", section 3.3),
 * a fork with copy-on-write, the precondition checks and the argument errors
 * of the device calls. Prints one line per result for the test to compare. */
#include <stdio.h>

#include "pagedkv.h"

static int failures = 0;

static void expect(int cond, const char* what) {
  printf("%s %s\n", cond ? "ok" : "FAIL", what);
  if (!cond) ++failures;
}

int main(void) {
  const int32_t free_order[8] = {7, 1, 3, 0, 2, 4, 5, 6};
  const int32_t prompt[7] = {11, 12, 13, 14, 15, 16, 17};
  pa_alloc* a = NULL;
  int64_t slots[7];
  int64_t slot = 0;
  int32_t table[8], n = 0, cached = -1, rc = -1, src_dst[2 * 4], ncopy = 0;

  expect(pa_version() > 0, "version");
  expect(pa_alloc_create(8, 4, free_order, &a) == PA_OK && a != NULL, "create");
  expect(pa_alloc_allocate(a, 1, prompt, 7, &cached, slots) == PA_OK && cached == 0, "allocate");
  expect(pa_alloc_block_table(a, 1, table, 8, &n) == PA_OK && n == 2 && table[0] == 7 &&
             table[1] == 1, "table after prompt = 7, 1");
  expect(slots[0] == 28 && slots[3] == 31 && slots[4] == 4 && slots[6] == 6,
         "prompt slots = 28..31, 4..6");
  expect(pa_alloc_append_slot(a, 1, 18, &slot) == PA_OK && slot == 7, "first decode slot = 7");
  expect(pa_alloc_append_slot(a, 1, 19, &slot) == PA_OK && slot == 12, "second decode slot = 12");
  expect(pa_alloc_block_table(a, 1, table, 8, &n) == PA_OK && n == 3 && table[2] == 3,
         "table after decode = 7, 1, 3");

  /* fork: the child shares every block; its append into the shared, partly
   * filled last block moves it to a new block and queues the copy */
  expect(pa_alloc_fork(a, 1, 2) == PA_OK, "fork");
  expect(pa_alloc_ref_count(a, 3, &rc) == PA_OK && rc == 2, "shared last block has count 2");
  expect(pa_alloc_append_slot(a, 2, 20, &slot) == PA_OK && slot / 4 != 3, "child copies on write");
  expect(pa_alloc_take_copies(a, src_dst, 4, &ncopy) == PA_OK && ncopy == 1 && src_dst[0] == 3 &&
             src_dst[1] == slot / 4, "one copy queued: 3 -> the child's new block");
  expect(pa_alloc_free(a, 2) == PA_OK && pa_alloc_free(a, 1) == PA_OK && pa_alloc_num_free(a) == 8,
         "every block free again");
  expect(pa_alloc_free(a, 1) == PA_ERR_STATE, "freeing twice is refused");
  pa_alloc_destroy(a);

  /* precondition checks on host arrays (the pool's memory is not touched) */
  pa_pool pool = {NULL, NULL, 8, 2, 4, 64, PA_BF16, 1.0f, 1.0f};
  const int32_t tables[2 * 3] = {7, 1, 3, 0, 2, 0};
  int32_t lens[2] = {9, 5};
  expect(pa_check_batch(&pool, tables, 3, lens, 2) == PA_OK, "batch checks out");
  lens[1] = 13;
  expect(pa_check_batch(&pool, tables, 3, lens, 2) == PA_ERR_INVALID, "too long a sequence refused");
  const int64_t dup[3] = {5, -1, 5};
  expect(pa_check_slots(&pool, dup, 3) == PA_ERR_INVALID, "a slot named twice refused");
  expect(pa_last_error() != NULL && pa_last_error()[0] != '\0', "the refusal is explained");

  /* device calls refuse bad arguments before any launch */
  expect(pa_decode(NULL, NULL, &pool, tables, 3, lens, 2, 4, 0.125f, 0, NULL, 0, NULL) ==
             PA_ERR_INVALID, "decode with NULL buffers refused");
  expect(pa_cache_write(NULL, NULL, NULL, NULL, 1, NULL) == PA_ERR_INVALID,
         "cache write without a pool refused");

  /* workspace sizes: the multi-row decode of 4 rows x 8 query heads per KV
     head (32 columns) takes, per work slice, two 32-row slots of bf16
     partials and (max, denominator) records, and one split record */
  expect(pa_attention_mixed_workspace_bytes(0, 256, 64, 8, 128, 4, 10) ==
             (size_t)(2 * 10 * 32 * 128 * 2 + 2 * 10 * 32 * 8 + 10 * 16),
         "multi-row workspace size");
  expect(pa_attention_mixed_workspace_bytes(0, 8, 6, 4, 128, 4, 10) == 0,
         "workspace size of 6 query heads over 4 KV heads is 0");
  expect(pa_decode_workspace_bytes(64, 40, 40, 128, 100) > 0, "decode workspace size");
  printf("%d failures\n", failures);
  return failures != 0;
}
