/* Host validation under extreme sizes: every entry point is called with each
 * of its size arguments in turn set to 0, -1, INT_MIN and INT_MAX (the other
 * arguments valid, pointers fake and 16-byte aligned), and with the extreme
 * values that overflow the size products. Built with the sanitizers by the
 * test suite, so signed overflow or an out-of-bounds access in the checks ends
 * the run. A call that passes validation reaches the launch, which fails
 * where there is no GPU (the suite runs this program only there), so no call
 * may return ATTN_OK. Exits 0 when none does. */
#include <limits.h>
#include <stdint.h>
#include <stdio.h>

#include "attn.h"

static void* F = (void*)(uintptr_t)(1u << 20);
static const int EXT[4] = {0, -1, INT_MIN, INT_MAX};
static int bad = 0, calls = 0;

static void expect_error(int st, const char* what, int arg, int val) {
  ++calls;
  if (st == ATTN_OK) {
    fprintf(stderr, "%s: argument %d = %d returned ATTN_OK\n", what, arg, val);
    bad = 1;
  }
}

#define SWEEP(NAME, NARGS, CALL)                                  \
  for (int a = 0; a < NARGS; ++a)                                 \
    for (int e = 0; e < 4; ++e) {                                 \
      int v[NARGS];                                               \
      for (int i = 0; i < NARGS; ++i) v[i] = base[i];             \
      v[a] = EXT[e];                                              \
      expect_error(CALL, NAME, a, EXT[e]);                        \
    }

int main(void) {
  {
    /* B, H, L, D, causal, dtype */
    const int base[6] = {2, 3, 100, 128, 1, ATTN_BF16};
    SWEEP("attn_prefill", 6,
          attn_prefill(F, F, F, F, NULL, v[0], v[1], v[2], v[3], v[4], 0.1f, v[5], NULL));
  }
  {
    /* B, H, q_len, D, num_blocks, width, block_size, causal, splits, dtype */
    const int base[10] = {2, 4, 1, 128, 10, 8, 16, 1, 2, ATTN_BF16};
    SWEEP("attn_paged_decode", 10,
          attn_paged_decode(F, F, F, F, F, F, NULL, v[0], v[1], v[2], v[3], v[4], v[5], v[6],
                            v[7], 0.1f, v[8], NULL, 0, v[9], NULL));
    SWEEP("attn_paged_decode_gqa", 10,
          attn_paged_decode_gqa(F, F, F, F, F, F, NULL, v[0], v[1], 2, v[2], v[3], v[4],
                                v[5], v[6], v[7], 0.1f, v[8], NULL, 0, v[9], NULL));
    SWEEP("attn_paged_decode_fp8", 10,
          attn_paged_decode_fp8(F, F, F, F, F, F, F, F, NULL, v[0], v[1], v[1], v[2], v[3], v[4],
                                v[5], v[6], v[7], 0.1f, v[8], NULL, (size_t)v[9] * 0, NULL));
  }
  {
    /* B, H, q_len, D, num_blocks, width, block_size, causal, dtype */
    const int base[9] = {2, 4, 64, 128, 10, 8, 16, 1, ATTN_BF16};
    SWEEP("attn_paged_prefill", 9,
          attn_paged_prefill(F, F, F, F, F, F, NULL, v[0], v[1], v[2], v[3], v[4], v[5], v[6],
                             v[7], 0.1f, v[8], NULL));
  }
  {
    /* B, H, total_q, max_q_len, D, num_blocks, width, block_size */
    const int base[8] = {2, 4, 40, 30, 128, 64, 8, 16};
    SWEEP("attn_paged_prefill_varlen", 8,
          attn_paged_prefill_varlen(F, F, F, F, F, F, F, NULL, v[0], v[1], v[2], v[3], v[4],
                                    v[5], v[6], v[7], 1, 0.1f, ATTN_BF16, NULL));
  }
  {
    /* B, H, q_len, S, D */
    const int base[5] = {2, 3, 1, 4, 128};
    SWEEP("attn_lse_merge", 5,
          attn_lse_merge(F, F, F, NULL, v[0], v[1], v[2], v[3], v[4], ATTN_BF16, NULL));
  }
  {
    /* B, H, D, num_blocks, width, max_seq_len */
    const int base[6] = {2, 3, 128, 10, 8, 64};
    SWEEP("attn_paged_gather", 6,
          attn_paged_gather(F, F, F, F, v[0], v[1], v[2], v[3], v[4], v[5], NULL));
  }
  {
    /* B, H, n_new, D, num_blocks, width, block_size */
    const int base[7] = {2, 3, 5, 128, 10, 8, 16};
    SWEEP("attn_paged_append", 7,
          attn_paged_append(F, F, F, F, F, F, v[0], v[1], v[2], v[3], v[4], v[5], v[6],
                            ATTN_BF16, NULL));
    SWEEP("attn_paged_append_fp8", 7,
          attn_paged_append_fp8(F, F, F, F, F, F, F, F, v[0], v[1], v[2], v[3], v[4], v[5],
                                v[6], NULL));
  }
  {
    /* n, num_blocks, H, D */
    const int base[4] = {3, 10, 4, 128};
    SWEEP("attn_paged_copy_blocks", 4,
          attn_paged_copy_blocks(F, F, F, F, v[0], v[1], v[2], v[3], ATTN_BF16, NULL));
    SWEEP("attn_paged_copy_blocks_fp8", 4,
          attn_paged_copy_blocks_fp8(F, F, F, F, F, F, v[0], v[1], v[2], v[3], NULL));
  }
  {
    /* checks: B, min_len / n_new, num_blocks, width */
    const int base[4] = {3, 1, 10, 8};
    SWEEP("attn_paged_check_tables", 4,
          attn_paged_check_tables(F, F, v[0], v[1], v[2], v[3], F, NULL));
    SWEEP("attn_paged_check_append", 4,
          attn_paged_check_append(F, F, v[0], v[1], v[2], v[3], F, NULL));
    SWEEP("attn_paged_check_ragged", 4,
          attn_paged_check_ragged(F, F, v[0], v[1], v[2], F, NULL));
    SWEEP("attn_paged_check_ids", 4, attn_paged_check_ids(F, F, v[0], v[1], F, NULL));
  }
  /* size queries: non-positive sizes give 0; huge ones give the exact byte
   * count, never a wrapped one (4 bytes x (D + 1) per partial row) */
  for (int e = 0; e < 4; ++e) {
    const int x = EXT[e];
    ++calls;
    const size_t got_b = attn_paged_workspace_bytes(x, 40, 5, 128, 2048, 16);
    const size_t got_h = attn_paged_workspace_bytes(4, x, 5, 128, 2048, 16);
    const size_t got_g = attn_paged_gqa_workspace_bytes(4, 40, x, 5, 128, 2048, 16);
    const size_t got_w = attn_paged_workspace_bytes(4, 40, 5, 128, x, 0);
    const unsigned __int128 row = (unsigned __int128)4 * 129;
    const size_t want_b = x > 0 ? (size_t)(row * (unsigned)x * 40 * 5 * 16) : 0;
    const size_t want_h = x > 0 ? (size_t)(row * 4 * (unsigned)x * 5 * 16) : 0;
    if (got_b != want_b || got_h != want_h || got_g != 0 ||
        got_w > (size_t)4 * 4 * 40 * 5 * 64 * 129) {
      fprintf(stderr, "workspace size query with %d: %zu %zu %zu %zu\n", x, got_b, got_h, got_g,
              got_w);
      bad = 1;
    }
  }
  /* overflowing products on otherwise valid sizes */
  expect_error(attn_prefill(F, F, F, F, NULL, INT_MAX, INT_MAX, INT_MAX, 128, 1, 0.1f, ATTN_BF16,
                            NULL), "attn_prefill product", -1, 0);
  expect_error(attn_paged_decode(F, F, F, F, F, F, NULL, 65535, 65535, 16, 128, INT_MAX, INT_MAX,
                                 16, 1, 0.1f, 1, NULL, 0, ATTN_BF16, NULL),
               "attn_paged_decode product", -1, 0);
  expect_error(attn_lse_merge(F, F, F, NULL, INT_MAX, INT_MAX, 16, 1024, 128, ATTN_F32, NULL),
               "attn_lse_merge product", -1, 0);
  if (bad) return 1;
  printf("validation_edges ok: %d calls\n", calls);
  return 0;
}
