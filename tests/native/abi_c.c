/* The C ABI from plain C99 (no Python, no GPU calls): build info, the
 * decode plan and workspace queries, validation errors before any device
 * work, and a serving-style host flow -- allocator, block manager with a
 * shared prefix found by the prefix cache, fork and copy-on-write pairs,
 * exported block tables.  Exits non-zero on the first failed check. */
#include <stddef.h>
#include <stdio.h>
#include <string.h>

#include "pa.h"

static int g_fail = 0;
#define CHECK(cond)                                                  \
  do {                                                               \
    if (!(cond)) {                                                   \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      g_fail = 1;                                                    \
    }                                                                \
  } while (0)

int main(void) {
  CHECK(strstr(pa_build_info(), "gfx950") != NULL);
  /* struct layouts, for bindings in other languages */
  printf("layout pa_tensor %zu %zu %zu %zu %zu %zu\n", sizeof(pa_tensor),
         offsetof(pa_tensor, dtype), offsetof(pa_tensor, ndim), offsetof(pa_tensor, shape),
         offsetof(pa_tensor, stride), offsetof(pa_tensor, scale));
  printf("layout pa_launch %zu %zu %zu %zu %zu %zu\n", sizeof(pa_launch),
         offsetof(pa_launch, workspace), offsetof(pa_launch, workspace_bytes),
         offsetof(pa_launch, partition_tokens), offsetof(pa_launch, path),
         offsetof(pa_launch, error_flags));
  CHECK(PA_NUM_FLAGS == 4 && PA_FLAG_QUERY_START == 3);

  /* decode plan: 32 sequences, 32 heads, d 128, bs 16, up to 2048 tokens */
  pa_decode_plan_info info;
  CHECK(pa_decode_plan(32, 32, 32, 128, 16, 128, 0, &info) == PA_OK);
  CHECK(info.schedule == PA_SCHEDULE_BALANCED);
  CHECK(info.workspace_bytes == pa_decode_workspace_bytes(32, 32, 32, 128, 16, 128, 0));
  CHECK(pa_decode_plan(32, 32, 32, 96, 16, 128, 0, &info) == PA_ERR_UNSUPPORTED);

  /* validation fails before any device work */
  CHECK(pa_decode(NULL, NULL, NULL, NULL, NULL, NULL, 0.1f, 16, 8, NULL) == PA_ERR_INVALID_ARG);
  CHECK(strlen(pa_last_error()) > 0);
  CHECK(pa_prefill(NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, 0.1f, 16, 8, NULL) == PA_ERR_INVALID_ARG);

  /* host flow: 2-token blocks, a 4-token prompt cached, a second request
   * with the same prompt reuses its blocks */
  pa_allocator* a = pa_alloc_create(16, NULL);
  CHECK(a != NULL);
  pa_block_manager* m = pa_bm_create(a, 2);
  pa_prefix_cache* pc = pa_pc_create(a, 2);
  CHECK(m != NULL && pc != NULL);
  const int32_t prompt[4] = {11, 12, 13, 14};
  int32_t blocks[2];
  CHECK(pa_pc_match(pc, prompt, 4, blocks, 2) == 0); /* empty cache */
  CHECK(pa_bm_add_sequence(m, 1, NULL, 0, 0) == PA_OK);
  for (int t = 0; t < 4; ++t) {
    int64_t slot;
    int32_t src, dst;
    CHECK(pa_bm_append_slot(m, 1, &slot, &src, &dst) == PA_OK);
    CHECK(src == -1 && dst == -1);
  }
  int64_t ids[2] = {1, 2};
  int32_t tables[2 * 4], lens[2];
  CHECK(pa_bm_export(m, ids, 1, 4, tables, lens) == PA_OK);
  CHECK(lens[0] == 4);
  CHECK(pa_pc_insert(pc, prompt, 4, tables, 2) == 2);
  CHECK(pa_pc_size(pc) == 2);
  /* second request: the prefix cache returns the same two blocks */
  CHECK(pa_pc_match(pc, prompt, 4, blocks, 2) == 2);
  CHECK(blocks[0] == tables[0] && blocks[1] == tables[1]);
  CHECK(pa_bm_add_sequence(m, 2, blocks, 2, 4) == PA_OK);
  /* the caller's match references are released once the manager holds its own */
  CHECK(pa_alloc_decref(a, blocks[0]) == PA_OK && pa_alloc_decref(a, blocks[1]) == PA_OK);
  CHECK(pa_alloc_refcount(a, blocks[0]) == 3); /* sequence 1, sequence 2, cache */
  CHECK(pa_bm_export(m, ids, 2, 4, tables, lens) == PA_OK);
  CHECK(lens[1] == 4 && tables[4] == tables[0] && tables[5] == tables[1]);
  /* fork, then the child's next token goes to a fresh block (the shared
   * blocks are full), no copy needed */
  CHECK(pa_bm_fork(m, 2, 3) == PA_OK);
  int64_t slot;
  int32_t src, dst;
  CHECK(pa_bm_append_slot(m, 3, &slot, &src, &dst) == PA_OK);
  CHECK(src == -1 && pa_bm_seq_len(m, 3) == 5);
  /* parent appends into a new block, then the child writing its own
   * partial last block needs no copy either */
  CHECK(pa_bm_append_slot(m, 2, &slot, &src, &dst) == PA_OK);
  /* release everything: only the cache's references remain, then evict */
  CHECK(pa_bm_free_sequence(m, 1) == PA_OK);
  CHECK(pa_bm_free_sequence(m, 2) == PA_OK);
  CHECK(pa_bm_free_sequence(m, 3) == PA_OK);
  CHECK(pa_alloc_num_free(a) == 14);
  CHECK(pa_pc_evict(pc, 16) == 2);
  CHECK(pa_alloc_num_free(a) == 16);
  pa_pc_destroy(pc);
  pa_bm_destroy(m);
  pa_alloc_destroy(a);
  if (!g_fail) printf("abi ok\n");
  return g_fail;
}
