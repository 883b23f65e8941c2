/* Random sequences of block-allocator operations (append, fork, release),
 * each followed by a check of the allocator's invariants through its C ABI:
 * every live table entry is a valid id, a sequence holds ceil(len / 16)
 * blocks, a block's reference count equals the number of table entries
 * naming it, the free count equals the number of unreferenced blocks, and a
 * failing call changes nothing. Built with the sanitizers by the test suite,
 * so an out-of-bounds access or undefined behaviour in the allocator ends the
 * run. Exits 0 when every check holds. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "attn.h"

#define NB 64
#define NS 8
#define W 16

#define CHECK(cond)                                                      \
  do {                                                                   \
    if (!(cond)) {                                                       \
      fprintf(stderr, "check failed at line %d (step %d): %s\n", __LINE__, step, #cond); \
      return 1;                                                          \
    }                                                                    \
  } while (0)

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static int rnd(int n) {
  rng = rng * 6364136223846793005ull + 1442695040888963407ull;
  return (int)((rng >> 33) % (uint64_t)n);
}

static int snapshot(const attn_kv_cache* c, int32_t* tab, int32_t* lens, int32_t* refs) {
  if (attn_kv_cache_export(c, tab, lens) != ATTN_OK) return -1;
  for (int b = 0; b < NB; ++b) refs[b] = attn_kv_cache_block_refs(c, b);
  return attn_kv_cache_free_blocks(c);
}

int main(void) {
  int step = -1;
  attn_kv_cache* c = attn_kv_cache_create(NB, NS, W);
  CHECK(c != NULL);
  CHECK(attn_kv_cache_create(0, NS, W) == NULL && attn_kv_cache_create(NB, -1, W) == NULL);
  int32_t tab[NS * W], lens[NS], refs[NB];
  int32_t tab0[NS * W], lens0[NS], refs0[NB];
  int n_ok = 0, n_err = 0, n_cow = 0;
  for (step = 0; step < 20000; ++step) {
    const int free0 = snapshot(c, tab0, lens0, refs0);
    CHECK(free0 >= 0);
    const int op = rnd(10);
    int st;
    int32_t src = -7, dst = -7;
    int ncp = -1;
    if (op < 6) {
      const int seq = rnd(NS + 1) - (rnd(50) == 0);  /* now and then out of range */
      const int n = rnd(41) - (rnd(40) == 0);         /* now and then negative */
      st = attn_kv_cache_append(c, seq, n, &src, &dst, rnd(20) == 0 ? 0 : 1, &ncp);
      if (st == ATTN_OK && ncp == 1) {
        ++n_cow;
        CHECK(src != dst && src >= 0 && src < NB && dst >= 0 && dst < NB);
        CHECK(attn_kv_cache_block_refs(c, dst) == 1);
      }
    } else if (op < 8) {
      st = attn_kv_cache_fork(c, rnd(NS), rnd(NS));
    } else {
      st = attn_kv_cache_release(c, rnd(NS + 1));
    }
    const int fr = snapshot(c, tab, lens, refs);
    CHECK(fr >= 0);
    if (st != ATTN_OK) {
      ++n_err;
      /* a failing call changes nothing */
      CHECK(fr == free0);
      CHECK(memcmp(tab, tab0, sizeof tab) == 0 && memcmp(lens, lens0, sizeof lens) == 0);
      CHECK(memcmp(refs, refs0, sizeof refs) == 0);
      continue;
    }
    ++n_ok;
    int count[NB];
    memset(count, 0, sizeof count);
    for (int s = 0; s < NS; ++s) {
      CHECK(lens[s] >= 0 && lens[s] <= 16 * W);
      CHECK(attn_kv_cache_length(c, s) == lens[s]);
      const int used = (lens[s] + 15) / 16;
      for (int j = 0; j < W; ++j) {
        const int id = tab[s * W + j];
        if (j < used) {
          CHECK(id >= 0 && id < NB);
          ++count[id];
        } else {
          CHECK(id == -1);
        }
      }
    }
    int n_free = 0;
    for (int b = 0; b < NB; ++b) {
      CHECK(refs[b] == count[b]);
      n_free += refs[b] == 0;
    }
    CHECK(n_free == fr);
  }
  CHECK(attn_kv_cache_block_refs(c, NB) < 0 && attn_kv_cache_length(c, NS) < 0);
  attn_kv_cache_destroy(c);
  attn_kv_cache_destroy(NULL);
  printf("alloc_fuzz ok: %d calls succeeded, %d refused, %d copy-on-write\n", n_ok, n_err, n_cow);
  return 0;
}
