/* Calls the library through its C header from C: version, status strings,
 * host-side argument validation (nothing reaches a device), and the host block
 * allocator (pure host code). Exits 0 when every check holds; prints the first
 * failing check otherwise. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "attn.h"

#define CHECK(cond)                                                  \
  do {                                                               \
    if (!(cond)) {                                                   \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      return 1;                                                      \
    }                                                                \
  } while (0)

int main(void) {
  CHECK(attn_version() == ATTN_VERSION);
  CHECK(strcmp(attn_status_string(ATTN_OK), "ok") == 0);
  CHECK(strcmp(attn_status_string(ATTN_ERR_NO_BLOCKS), "unknown status") != 0);

  /* validation fails before any launch: fake, aligned, never dereferenced */
  void* fake = (void*)(uintptr_t)(1u << 20);
  CHECK(attn_prefill(NULL, fake, fake, fake, NULL, 1, 1, 64, 128, 1, 0.1f, ATTN_BF16, NULL) ==
        ATTN_ERR_NULL_PTR);
  CHECK(attn_prefill(fake, fake, fake, fake, NULL, 1, 1, 64, 96, 1, 0.1f, ATTN_BF16, NULL) ==
        ATTN_ERR_UNSUPPORTED);
  CHECK(attn_paged_decode(fake, fake, fake, fake, fake, fake, NULL, 1, 1, 1, 128, 4, 4, 32, 1,
                          0.1f, 0, NULL, 0, ATTN_BF16, NULL) == ATTN_ERR_UNSUPPORTED);
  CHECK(attn_paged_workspace_bytes(4, 8, 1, 128, 64, 1) == 0);
  CHECK(attn_paged_workspace_bytes(4, 8, 1, 128, 64, 4) ==
        (size_t)4 * 4 * 8 * 1 * 4 * (128 + 1));

  /* the paging figure: A takes blocks 0, 1, 5, 7, 8 and B takes 2, 9 */
  attn_kv_cache* c = attn_kv_cache_create(11, 4, 8);
  CHECK(c != NULL);
  int32_t src[1], dst[1];
  int n = -1;
  const int steps[7][2] = {{0, 32}, {1, 16}, {2, 32}, {0, 16}, {3, 16}, {0, 32}, {1, 16}};
  for (int i = 0; i < 7; ++i) {
    CHECK(attn_kv_cache_append(c, steps[i][0], steps[i][1], src, dst, 1, &n) == ATTN_OK);
    CHECK(n == 0);
  }
  CHECK(attn_kv_cache_release(c, 2) == ATTN_OK);
  CHECK(attn_kv_cache_release(c, 3) == ATTN_OK);
  int32_t tables[4 * 8], lens[4];
  CHECK(attn_kv_cache_export(c, tables, lens) == ATTN_OK);
  const int32_t a[5] = {0, 1, 5, 7, 8}, b[2] = {2, 9};
  for (int i = 0; i < 5; ++i) CHECK(tables[i] == a[i]);
  for (int i = 0; i < 2; ++i) CHECK(tables[8 + i] == b[i]);
  CHECK(lens[0] == 80 && lens[1] == 32 && lens[2] == 0);
  CHECK(attn_kv_cache_free_blocks(c) == 4);

  /* fork mid-block, then copy-on-write on the child's first append */
  CHECK(attn_kv_cache_append(c, 2, 20, src, dst, 1, &n) == ATTN_OK && n == 0);
  CHECK(attn_kv_cache_fork(c, 2, 3) == ATTN_OK);
  CHECK(attn_kv_cache_append(c, 3, 1, src, dst, 1, &n) == ATTN_OK);
  CHECK(n == 1 && src[0] != dst[0]);
  CHECK(attn_kv_cache_block_refs(c, src[0]) == 1 && attn_kv_cache_block_refs(c, dst[0]) == 1);
  CHECK(attn_kv_cache_append(c, 0, 1000, src, dst, 1, &n) == ATTN_ERR_BAD_SHAPE);
  CHECK(attn_kv_cache_append(c, 1, 60, src, dst, 1, &n) == ATTN_ERR_NO_BLOCKS);  /* 1 block free */
  attn_kv_cache_destroy(c);
  printf("abi_check ok\n");
  return 0;
}
