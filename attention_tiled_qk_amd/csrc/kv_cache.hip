// Host-side block allocator of the paged KV cache (no device code).
//
// The pool's physical blocks are handed out on demand as sequences grow, one
// 16-token block at a time, and returned when a sequence is released ([P3],
// Continuous Batching + PagedAttention item: allocate when the last block is
// full, free everything when the request ends). Blocks carry reference counts
// so that a forked sequence shares its parent's blocks -- e.g. a common prompt
// prefix -- and a shared block is copied before either owner writes into it
// ([P4], the fanzheng.org survey's subsection on paged memory management:
// reference-counted blocks, copy-on-write; [P1] §3.2 and [P2] §二, requests
// with a common prefix share its pages).
//
// The allocator only does bookkeeping: it reports the (source, destination)
// block copies that copy-on-write needs, the caller runs them on the device
// (attn_paged_copy_blocks) and uploads the tables (attn_kv_cache_export)
// before appending tokens (attn_paged_append) or running attention.
#include <cstdint>
#include <new>
#include <vector>

#include "../../include/attn.h"

struct attn_kv_cache {
  int num_blocks = 0;
  int max_seqs = 0;
  int max_blocks = 0;
  std::vector<int32_t> free_ids;                // stack of free physical blocks
  std::vector<int32_t> refs;                    // reference count per physical block
  std::vector<std::vector<int32_t>> tables;     // per sequence: logical -> physical
  std::vector<int32_t> lens;                    // tokens per sequence
};

namespace {

bool valid_seq(const attn_kv_cache* c, int seq) { return c && seq >= 0 && seq < c->max_seqs; }

}  // namespace

extern "C" {

attn_kv_cache* attn_kv_cache_create(int num_blocks, int max_seqs, int max_blocks_per_seq) {
  if (num_blocks <= 0 || max_seqs <= 0 || max_blocks_per_seq <= 0) return nullptr;
  attn_kv_cache* c = new (std::nothrow) attn_kv_cache;
  if (!c) return nullptr;
  c->num_blocks = num_blocks;
  c->max_seqs = max_seqs;
  c->max_blocks = max_blocks_per_seq;
  c->free_ids.reserve(num_blocks);
  // lowest ids are handed out first
  for (int i = num_blocks - 1; i >= 0; --i) c->free_ids.push_back(i);
  c->refs.assign(num_blocks, 0);
  c->tables.assign(max_seqs, {});
  c->lens.assign(max_seqs, 0);
  return c;
}

void attn_kv_cache_destroy(attn_kv_cache* cache) { delete cache; }

int attn_kv_cache_append(attn_kv_cache* c, int seq, int n_tokens, int32_t* copy_src,
                         int32_t* copy_dst, int max_copies, int* n_copies) {
  if (!valid_seq(c, seq) || n_tokens < 0 || !n_copies) return ATTN_ERR_BAD_SHAPE;
  *n_copies = 0;
  if (n_tokens == 0) return ATTN_OK;
  std::vector<int32_t>& tab = c->tables[seq];
  const long long len = c->lens[seq];
  const long long new_len = len + n_tokens;
  const long long need = (new_len + ATTN_BLOCK_SIZE - 1) / ATTN_BLOCK_SIZE;
  if (need > c->max_blocks) return ATTN_ERR_BAD_SHAPE;
  // the partly filled last block receives tokens: copy it first if it is shared
  const bool cow = (len % ATTN_BLOCK_SIZE) != 0 && c->refs[tab.back()] > 1;
  if (cow && (max_copies < 1 || !copy_src || !copy_dst)) return ATTN_ERR_WORKSPACE;
  const long long fresh = need - (long long)tab.size() + (cow ? 1 : 0);
  if (fresh > (long long)c->free_ids.size()) return ATTN_ERR_NO_BLOCKS;  // nothing changed
  if (cow) {
    const int32_t shared = tab.back();
    const int32_t own = c->free_ids.back();
    c->free_ids.pop_back();
    c->refs[shared] -= 1;
    c->refs[own] = 1;
    tab.back() = own;
    copy_src[0] = shared;
    copy_dst[0] = own;
    *n_copies = 1;
  }
  while ((long long)tab.size() < need) {
    const int32_t id = c->free_ids.back();
    c->free_ids.pop_back();
    c->refs[id] = 1;
    tab.push_back(id);
  }
  c->lens[seq] = (int32_t)new_len;
  return ATTN_OK;
}

int attn_kv_cache_fork(attn_kv_cache* c, int parent, int child) {
  if (!valid_seq(c, parent) || !valid_seq(c, child) || parent == child) return ATTN_ERR_BAD_SHAPE;
  if (c->lens[child] != 0 || !c->tables[child].empty()) return ATTN_ERR_BAD_SHAPE;
  c->tables[child] = c->tables[parent];
  for (int32_t id : c->tables[child]) c->refs[id] += 1;
  c->lens[child] = c->lens[parent];
  return ATTN_OK;
}

int attn_kv_cache_release(attn_kv_cache* c, int seq) {
  if (!valid_seq(c, seq)) return ATTN_ERR_BAD_SHAPE;
  for (int32_t id : c->tables[seq]) {
    c->refs[id] -= 1;
    if (c->refs[id] == 0) c->free_ids.push_back(id);
  }
  c->tables[seq].clear();
  c->lens[seq] = 0;
  return ATTN_OK;
}

int attn_kv_cache_length(const attn_kv_cache* c, int seq) {
  return valid_seq(c, seq) ? c->lens[seq] : ATTN_ERR_BAD_SHAPE;
}

int attn_kv_cache_free_blocks(const attn_kv_cache* c) {
  return c ? (int)c->free_ids.size() : ATTN_ERR_NULL_PTR;
}

int attn_kv_cache_block_refs(const attn_kv_cache* c, int block) {
  if (!c) return ATTN_ERR_NULL_PTR;
  if (block < 0 || block >= c->num_blocks) return ATTN_ERR_BAD_SHAPE;
  return c->refs[block];
}

int attn_kv_cache_export(const attn_kv_cache* c, int32_t* block_tables, int32_t* seq_lens) {
  if (!c || !block_tables || !seq_lens) return ATTN_ERR_NULL_PTR;
  for (int s = 0; s < c->max_seqs; ++s) {
    int32_t* row = block_tables + (size_t)s * c->max_blocks;
    const std::vector<int32_t>& tab = c->tables[s];
    for (int i = 0; i < c->max_blocks; ++i) row[i] = i < (int)tab.size() ? tab[i] : -1;
    seq_lens[s] = c->lens[s];
  }
  return ATTN_OK;
}

}  // extern "C"
