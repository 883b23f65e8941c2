/*
 * attn.h -- C ABI of the gfx950 (MI355X) tiled-attention library.
 *
 * Exact attention O = softmax(scale * Q K^T + mask) V computed IO-aware: the
 * score matrix is formed tile by tile on chip and folded into a running row
 * maximum m and exponential sum l (online softmax), so it never reaches HBM.
 * Sources, cited by page and section:
 *   [P1] iopencloud.com, "大模型推理加速技术全景：从FlashAttention到Speculative
 *        Decoding": §2.1 standard attention, §2.2 tiling and online softmax,
 *        §3.2 PagedAttention (16-token block pool and per-request page tables).
 *   [P2] ybb.press/llm-inference/15723.html: §一 the scaled dot-product
 *        attention formula softmax(QK^T / sqrt(d_k)) V.
 *   [P3] lowentro.cn notes "推理加速技术": the FlashAttention core-idea item,
 *        the FlashAttention-2 item, the FlashDecoding item (split the key range
 *        across workgroups, then a cross-split reduction kernel), and the
 *        Continuous Batching + PagedAttention item (the kernel receives each
 *        request's block table and reads only valid blocks; blocks are
 *        allocated as a request grows and freed when it ends).
 *   [P4] fanzheng.org inference survey, section on KV-cache runtime
 *        management and reuse, subsection on paged memory management:
 *        physical blocks carry reference counts, sequences that share them
 *        copy on write.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller. The library
 *     never allocates, frees or synchronises; it enqueues kernels on `stream`
 *     (a hipStream_t; NULL = the null stream) and returns. Results are ready
 *     when the stream reaches that point.
 *   - Layouts are dense, row-major, innermost dimension last, as stated per
 *     argument. Pointers must be 16-byte aligned.
 *   - dtype: ATTN_F32 = float32, ATTN_BF16 = bfloat16. Accumulation is float32.
 *   - Causal masking is bottom-right aligned: with Lq queries over Lk keys,
 *     query t sits at position Lk - Lq + t and sees keys 0 .. Lk - Lq + t.
 *   - lse outputs are the natural-log log-sum-exp of the scaled scores of each
 *     query row (float32); a row that sees no key gets -inf and a zero output.
 *   - Every argument is validated on the host before anything is enqueued. On
 *     error the call returns a negative ATTN_ERR_* code and enqueues nothing.
 *     Device-side contents are trusted: block ids outside [0, num_blocks) or
 *     seq_lens above max_blocks_per_seq * 16 are undefined behaviour;
 *     attn_paged_check_tables, _check_append, _check_ragged and _check_ids
 *     count such entries on the device.
 *   - Calls are stateless and re-entrant; calls on different streams may run
 *     concurrently if their output buffers do not overlap.
 */
#ifndef ATTN_TILED_QK_H
#define ATTN_TILED_QK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_VERSION 100 /* 1.0.0 */

enum attn_dtype { ATTN_F32 = 0, ATTN_BF16 = 1 };

enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_NULL_PTR = -1,    /* a required pointer is NULL */
  ATTN_ERR_BAD_SHAPE = -2,   /* a size is zero/negative or shapes disagree */
  ATTN_ERR_BAD_DTYPE = -3,   /* dtype not supported by this entry point */
  ATTN_ERR_UNSUPPORTED = -4, /* head_dim, q_len, block_size or split count outside the supported set */
  ATTN_ERR_MISALIGNED = -5,  /* a pointer is not 16-byte aligned */
  ATTN_ERR_WORKSPACE = -6,   /* workspace missing or smaller than attn_paged_workspace_bytes() */
  ATTN_ERR_OVERFLOW = -7,    /* an element count does not fit the kernels' 32/64-bit indexing */
  ATTN_ERR_HIP = -8,         /* the kernel launch itself failed (hipGetLastError) */
  ATTN_ERR_NO_BLOCKS = -9,   /* the block allocator has too few free blocks */
  ATTN_ERR_SCRATCH = -10     /* split-KV partials larger than ATTN_NOALLOC_SCRATCH_BYTES */
};

/* Largest query count per sequence accepted by attn_paged_decode. */
#define ATTN_PAGED_MAX_QLEN 16
/* Largest explicit split count accepted by attn_paged_decode. */
#define ATTN_PAGED_MAX_SPLITS 64
/* The only KV block size supported (tokens per physical block). */
#define ATTN_BLOCK_SIZE 16

/*
 * attn_prefill -- exact attention for a batch of full sequences
 *                 ([P1] §2.2 tiling + online softmax, [P2] §一 formula).
 *
 *   q, k, v : [B, H, L, D] of `dtype`, contiguous.
 *   o       : [B, H, L, D] of `dtype` (written). May not alias q, k or v.
 *   lse     : [B, H, L] float32 (written), or NULL to skip it.
 *   B, H, L : batch, heads, sequence length (>= 1).
 *   D       : head dimension, 64 or 128.
 *   causal  : 0 = full attention, 1 = causal (query i sees keys 0..i).
 *   scale   : multiplier of Q K^T (normally 1/sqrt(D)); finite.
 *   dtype   : ATTN_F32 or ATTN_BF16.
 * Returns ATTN_OK or a negative ATTN_ERR_* code.
 */
int attn_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int L, int D, int causal, float scale, int dtype,
                 void* stream);

/*
 * attn_paged_workspace_bytes -- size of the float32 scratch that
 * attn_paged_decode needs for `num_splits` split-KV partials ([P3]
 * FlashDecoding item: each split of the key range is attended on its own and
 * leaves a partial output and its log-sum-exp for the reduction): the
 * normalised partial outputs [B, H, q_len, S, D] and their lse
 * [B, H, q_len, S], 4 * B * H * q_len * S * (D + 1) bytes.
 * num_splits = 0 asks for the split count the library would choose itself,
 * which depends on the table width, so max_blocks_per_seq is an argument here
 * as well (it must be the max_blocks_per_seq of the decode call). Returns 0
 * when one split suffices (no workspace needed) and also for invalid
 * arguments.
 */
size_t attn_paged_workspace_bytes(int B, int H, int q_len, int D, int max_blocks_per_seq,
                                  int num_splits);

/*
 * attn_paged_decode -- attention of q_len new queries per sequence over a
 * PagedAttention KV cache ([P1] §3.2, [P3] block tables in the kernel), with
 * optional FlashDecoding split-KV ([P3]) and log-sum-exp merge.
 *
 *   q            : [B, H, q_len, D] bf16, contiguous.
 *   k_pool,
 *   v_pool       : [num_blocks, H, 16, D] bf16: physical block p, head h, slot s
 *                  holds the key/value of the token stored there.
 *   block_tables : [B, max_blocks_per_seq] int32 device array: entry n of row b
 *                  is the physical block holding tokens 16n .. 16n+15 of
 *                  sequence b. Entries at or past ceil(seq_lens[b] / 16) are
 *                  never read (pad with -1).
 *   seq_lens     : [B] int32 device array: the key count of each sequence,
 *                  INCLUDING its q_len new tokens (already written to the cache).
 *                  Must satisfy q_len <= seq_lens[b] <= max_blocks_per_seq * 16.
 *                  Slots past seq_len in the last block are never read.
 *   o            : [B, H, q_len, D] bf16 (written).
 *   lse          : [B, H, q_len] float32 (written), or NULL.
 *   q_len        : 1 .. ATTN_PAGED_MAX_QLEN (1 = decode; K+1 = speculative verify).
 *   D            : 128 (64 also accepted).
 *   block_size   : must be 16.
 *   causal       : 1 = bottom-right causal within the new tokens (query t sees
 *                  keys 0 .. seq_len - q_len + t); 0 = all seq_len keys.
 *   num_splits   : 0 = library's choice; else 1 .. ATTN_PAGED_MAX_SPLITS. With S
 *                  splits, sequence b's ceil(seq_len/16) blocks are cut into S
 *                  contiguous ranges of ceil(nb/S) blocks; each is attended
 *                  independently and the partials are merged.
 *   workspace    : device scratch of at least attn_paged_workspace_bytes(B, H,
 *                  q_len, D, max_blocks_per_seq, num_splits) bytes (may be NULL
 *                  when that is 0). Contents on entry are ignored.
 *   dtype        : must be ATTN_BF16.
 * Returns ATTN_OK or a negative ATTN_ERR_* code.
 */
int attn_paged_decode(const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_tables, const int32_t* seq_lens, void* o,
                      float* lse, int B, int H, int q_len, int D, int num_blocks,
                      int max_blocks_per_seq, int block_size, int causal, float scale,
                      int num_splits, void* workspace, size_t workspace_bytes, int dtype,
                      void* stream);

/* Longest sequence attn_paged_prefill accepts, in 16-token blocks (32768 keys). */
#define ATTN_PAGED_PREFILL_MAX_BLOCKS 2048

/*
 * attn_paged_prefill -- chunked prefill over a PagedAttention cache: the q_len
 * newest tokens of each sequence (already written to the cache) attend all of
 * its seq_lens[b] cached keys, read through its block table. This is the step
 * that splits a long prompt into chunks interleaved with decode ([P3], the
 * chunked-prefill and TTFT items), with the cache layout of [P1] §3.2; it runs
 * the tiled online-softmax prefill kernel with its K/V tiles gathered block by
 * block from the pool.
 *
 *   q, o         : [B, H, q_len, D] bf16 (query t of sequence b is its token
 *                  seq_lens[b] - q_len + t).
 *   k_pool,
 *   v_pool       : [num_blocks, H, 16, D] bf16.
 *   block_tables : [B, max_blocks_per_seq] int32 device; entries past
 *                  ceil(seq_lens[b] / 16) are never read.
 *   seq_lens     : [B] int32 device, q_len <= seq_lens[b] <= max_blocks_per_seq * 16.
 *   lse          : [B, H, q_len] float32 or NULL.
 *   D            : 64 or 128; block_size must be 16;
 *   max_blocks_per_seq <= ATTN_PAGED_PREFILL_MAX_BLOCKS.
 *   causal       : bottom-right (query t sees keys 0 .. seq_lens[b] - q_len + t).
 * Slots past seq_lens[b] are never read. Returns ATTN_OK or a negative
 * ATTN_ERR_* code.
 */
int attn_paged_prefill(const void* q, const void* k_pool, const void* v_pool,
                       const int32_t* block_tables, const int32_t* seq_lens, void* o, float* lse,
                       int B, int H, int q_len, int D, int num_blocks, int max_blocks_per_seq,
                       int block_size, int causal, float scale, int dtype, void* stream);

/*
 * attn_paged_prefill_varlen -- attn_paged_prefill for a ragged batch: each
 * sequence brings its own number of new query tokens, the way continuous
 * batching packs prompt chunks of different lengths (and single decode
 * tokens) into one step ([P3], the chunked-prefill and continuous-batching
 * items). Sequence b owns packed query tokens cu_q_lens[b] .. cu_q_lens[b+1]-1;
 * its t-th new token sits at position seq_lens[b] - q_len_b + t.
 *
 *   q, o         : [total_q, H, D] bf16, token-major (token i, head h at
 *                  (i * H + h) * D).
 *   lse          : [total_q, H] float32, or NULL.
 *   cu_q_lens    : [B + 1] int32 device, cu_q_lens[0] = 0, non-decreasing,
 *                  cu_q_lens[B] = total_q; q_len_b = cu_q_lens[b+1] - cu_q_lens[b]
 *                  may be 0 and must not exceed max_q_len or seq_lens[b]
 *                  (device contents are trusted, as for block tables).
 *   max_q_len    : the largest q_len_b (sizes the launch), <= total_q.
 *   Pools, tables, seq_lens, D, block_size, causal and scale as for
 *   attn_paged_prefill. Returns ATTN_OK or a negative ATTN_ERR_* code.
 */
int attn_paged_prefill_varlen(const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* block_tables, const int32_t* seq_lens,
                              const int32_t* cu_q_lens, void* o, float* lse, int B, int H,
                              int total_q, int max_q_len, int D, int num_blocks,
                              int max_blocks_per_seq, int block_size, int causal, float scale,
                              int dtype, void* stream);

/*
 * attn_paged_prefill_gqa -- attn_paged_prefill_varlen over pools with fewer
 * heads than the queries (grouped-query attention, [P3] TTFT item): H query
 * heads read Hkv KV heads, query head h reading KV head h / (H / Hkv)
 * (consecutive query heads form a group). Layouts and every other argument as
 * for attn_paged_prefill_varlen, except k_pool, v_pool: [num_blocks, Hkv, 16, D]
 * bf16. H must be a multiple of Hkv (else ATTN_ERR_BAD_SHAPE); with H == Hkv it
 * is attn_paged_prefill_varlen.
 */
int attn_paged_prefill_gqa(const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* block_tables, const int32_t* seq_lens,
                           const int32_t* cu_q_lens, void* o, float* lse, int B, int H, int Hkv,
                           int total_q, int max_q_len, int D, int num_blocks,
                           int max_blocks_per_seq, int block_size, int causal, float scale,
                           int dtype, void* stream);

/*
 * attn_paged_decode_gqa -- attn_paged_decode with grouped-query attention:
 * Hq query heads share Hkv KV heads, query head hq reading KV head
 * hq / (Hq / Hkv) (consecutive query heads form a group). The pools hold Hkv
 * heads; one wave serves all Hq / Hkv query heads of a group from a single read
 * of their K/V. [P3]'s item on cutting time-to-first-token names MQA and GQA
 * (fewer KV heads than query heads) as the way to shrink the KV cache; this is
 * that attention over the same paged cache. With Hq == Hkv it is
 * attn_paged_decode.
 *
 *   q, o         : [B, Hq, q_len, D] bf16.
 *   k_pool,
 *   v_pool       : [num_blocks, Hkv, 16, D] bf16.
 *   Hq, Hkv      : Hq a multiple of Hkv, and (Hq / Hkv) * q_len <= ATTN_PAGED_MAX_QLEN.
 *   lse          : [B, Hq, q_len] float32 or NULL.
 *   workspace    : at least attn_paged_gqa_workspace_bytes(B, Hq, Hkv, q_len, D,
 *                  max_blocks_per_seq, num_splits) bytes.
 *   Every other argument, the masking and the split semantics are those of
 *   attn_paged_decode. Returns ATTN_OK or a negative ATTN_ERR_* code
 *   (ATTN_ERR_BAD_SHAPE when Hkv does not divide Hq, ATTN_ERR_UNSUPPORTED when
 *   the group times q_len exceeds ATTN_PAGED_MAX_QLEN).
 */
int attn_paged_decode_gqa(const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* block_tables, const int32_t* seq_lens, void* o, float* lse,
                          int B, int Hq, int Hkv, int q_len, int D, int num_blocks,
                          int max_blocks_per_seq, int block_size, int causal, float scale,
                          int num_splits, void* workspace, size_t workspace_bytes, int dtype,
                          void* stream);

/* Size of the device scratch that attn_paged_decode_noalloc keeps per GPU. */
#define ATTN_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * attn_paged_decode_noalloc -- attn_paged_decode_gqa for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the split-KV partials go to a scratch
 * array of ATTN_NOALLOC_SCRATCH_BYTES that the library's code object reserves
 * on each GPU it is loaded onto, held until the process ends. The call itself
 * allocates nothing; its first call on a device looks the array's device
 * address up (hipGetSymbolAddress) for that device.
 *
 *   Arguments: those of attn_paged_decode_gqa without the workspace (Hkv == Hq
 *   for plain multi-head attention); the call runs on the current device, to
 *   which `stream` must belong. Outputs are identical to attn_paged_decode_gqa
 *   with the same num_splits.
 *   Returns ATTN_ERR_SCRATCH (before anything is enqueued) when the partials,
 *   attn_paged_gqa_workspace_bytes(B, Hq, Hkv, q_len, D, max_blocks_per_seq,
 *   num_splits) bytes, exceed ATTN_NOALLOC_SCRATCH_BYTES; ATTN_ERR_HIP when
 *   the device address cannot be obtained; otherwise as attn_paged_decode_gqa.
 *   All calls on one GPU share its scratch: calls that may overlap in time on
 *   one GPU (other streams, other host threads) race on it and must be
 *   serialised by the caller. Every call writes the partials it reads, so
 *   what an earlier call left there does not matter.
 */
int attn_paged_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* block_tables, const int32_t* seq_lens, void* o,
                              float* lse, int B, int Hq, int Hkv, int q_len, int D,
                              int num_blocks, int max_blocks_per_seq, int block_size, int causal,
                              float scale, int num_splits, int dtype, void* stream);

/*
 * attn_paged_gqa_workspace_bytes -- split-KV scratch size for
 * attn_paged_decode_gqa: 4 * B * Hq * q_len * S * (D + 1) bytes for the split
 * count S it will use (num_splits, or its own choice for 0, which depends on
 * B, Hkv and max_blocks_per_seq); 0 when one split suffices or the arguments
 * are invalid.
 */
size_t attn_paged_gqa_workspace_bytes(int B, int Hq, int Hkv, int q_len, int D,
                                      int max_blocks_per_seq, int num_splits);

/*
 * attn_lse_merge -- the FlashDecoding cross-split reduction ([P3]): combine S
 * softmax-normalised partial outputs with their log-sum-exps. For each row,
 * M = max_p lse_p, w_p = exp(lse_p - M), o = sum_p w_p o_p / sum_p w_p and
 * lse = M + log(sum_p w_p) -- the rescaling step of the online softmax of
 * [P1] §2.2 applied across splits. Rows whose partials are all -inf get o = 0
 * and lse = -inf.
 *
 *   o_part   : [B, H, q_len, S, D] float32.
 *   lse_part : [B, H, q_len, S] float32 (-inf marks an empty partial).
 *   o        : [B, H, q_len, D] of `dtype` (ATTN_F32 or ATTN_BF16), written.
 *   lse      : [B, H, q_len] float32, written, or NULL.
 *   S        : 1 .. 1024.  D: 64 or 128.
 * Returns ATTN_OK or a negative ATTN_ERR_* code.
 */
int attn_lse_merge(const float* o_part, const float* lse_part, void* o, float* lse,
                   int B, int H, int q_len, int S, int D, int dtype, void* stream);

/*
 * attn_paged_gather -- copy each sequence's cached rows out of a paged pool
 * into a contiguous tensor, through its block table ([P1] §3.2). Bit-exact
 * copy; used to check block-table indexing.
 *
 *   pool         : [num_blocks, H, 16, D] bf16.
 *   block_tables : [B, max_blocks_per_seq] int32 device.
 *   seq_lens     : [B] int32 device, each <= min(max_seq_len, max_blocks_per_seq*16).
 *   out          : [B, H, max_seq_len, D] bf16; rows t < seq_lens[b] are
 *                  written, the rest are left untouched.
 *   D            : 64 or 128.
 * Returns ATTN_OK or a negative ATTN_ERR_* code.
 */
int attn_paged_gather(const void* pool, const int32_t* block_tables, const int32_t* seq_lens,
                      void* out, int B, int H, int D, int num_blocks, int max_blocks_per_seq,
                      int max_seq_len, void* stream);

/*
 * attn_paged_check_tables -- count the entries of a paged-cache description
 * that the attention, append and gather calls would read out of range. Those
 * calls trust their tables ([P3] PagedAttention: a request's table lists the
 * only blocks its kernel reads), so this is a debugging aid to run before
 * them; it reads the tables only.
 *
 *   block_tables : [B, max_blocks_per_seq] int32 device.
 *   seq_lens     : [B] int32 device.
 *   min_len      : smallest valid length, >= 0 (the q_len of the call to check;
 *                  0 for a ragged prefill).
 *   bad          : 2 int32 device words, overwritten (not accumulated), each
 *                  saturating at INT32_MAX:
 *                  bad[0] = sequences with seq_lens[b] < min_len or
 *                           > max_blocks_per_seq * 16;
 *                  bad[1] = entries j < ceil(min(max(seq_lens[b], 0),
 *                           max_blocks_per_seq * 16) / 16) of row b (the ones
 *                           the calls read) outside [0, num_blocks).
 * One workgroup, enqueued on stream; the counts are valid once it completes.
 * Returns ATTN_OK or a negative ATTN_ERR_* code.
 */
int attn_paged_check_tables(const int32_t* block_tables, const int32_t* seq_lens, int B,
                            int min_len, int num_blocks, int max_blocks_per_seq, int32_t* bad,
                            void* stream);

/*
 * attn_paged_check_append -- attn_paged_check_tables for the append calls,
 * which read different entries: for each sequence, the entries covering its
 * n_new newest positions (those >= 0). Those must be -1 (the append places
 * nothing there) or inside [0, num_blocks).
 *   bad : 2 int32 device words, overwritten, each saturating at INT32_MAX:
 *         bad[0] = sequences with seq_lens[b] < 0 or > max_blocks_per_seq * 16;
 *         bad[1] = entries the append writes through that are < -1 or
 *                  >= num_blocks.
 * One workgroup on stream. Returns ATTN_OK or a negative ATTN_ERR_* code.
 */
int attn_paged_check_append(const int32_t* block_tables, const int32_t* seq_lens, int B, int n_new,
                            int num_blocks, int max_blocks_per_seq, int32_t* bad, void* stream);

/*
 * attn_paged_check_ragged -- checks the packed query offsets of a ragged
 * prefill call (attn_paged_prefill_varlen / _gqa), which trusts them:
 *   cu_q_lens : [B + 1] int32 device.  seq_lens : [B] int32 device.
 *   bad       : 2 int32 device words, overwritten, each saturating:
 *               bad[0] = offset errors: cu_q_lens[0] != 0, cu_q_lens[B] !=
 *                        total_q, and each decreasing step;
 *               bad[1] = sequences whose query count exceeds max_q_len or
 *                        their seq_lens[b].
 * One workgroup on stream. Returns ATTN_OK or a negative ATTN_ERR_* code.
 */
int attn_paged_check_ragged(const int32_t* cu_q_lens, const int32_t* seq_lens, int B, int total_q,
                            int max_q_len, int32_t* bad, void* stream);

/*
 * attn_paged_check_ids -- checks the block-id lists of a copy call
 * (attn_paged_copy_blocks / _fp8): bad[0] counts entries of src and bad[1]
 * entries of dst outside [0, num_blocks) (n ids each, int32 device arrays).
 * One workgroup on stream. Returns ATTN_OK or a negative ATTN_ERR_* code.
 */
int attn_paged_check_ids(const int32_t* src, const int32_t* dst, int n, int num_blocks,
                         int32_t* bad, void* stream);

/*
 * attn_paged_append -- write n_new new tokens of K and V per sequence into the
 * paged pools ([P1] §3.2 layout; [P3] Continuous Batching + PagedAttention:
 * the cache grows block by block). Token t of sequence b has position
 * p = seq_lens[b] - n_new + t and lands in physical block
 * block_tables[b][p / 16], slot p % 16 -- the exact inverse of the gather that
 * the attention calls perform. Bit-exact copy.
 *
 *   k_new, v_new : [B, H, n_new, D] bf16, contiguous.
 *   k_pool,
 *   v_pool       : [num_blocks, H, 16, D] bf16, written in place.
 *   block_tables : [B, max_blocks_per_seq] int32 device; the blocks covering
 *                  the new positions must already be assigned (see the
 *                  allocator below).
 *   seq_lens     : [B] int32 device, lengths INCLUDING the new tokens. A
 *                  sequence with seq_lens[b] < n_new places only the tokens
 *                  whose position is >= 0; table entries < 0 are skipped.
 *   D            : 64 or 128; block_size must be 16.
 * Sequences must not share a destination block (copy a shared block first,
 * attn_paged_copy_blocks). Returns ATTN_OK or a negative ATTN_ERR_* code.
 */
int attn_paged_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                      const int32_t* block_tables, const int32_t* seq_lens, int B, int H,
                      int n_new, int D, int num_blocks, int max_blocks_per_seq, int block_size,
                      int dtype, void* stream);

/*
 * attn_paged_copy_blocks -- copy-on-write support ([P4]): copy physical block
 * src[i] onto dst[i] (all H heads, all 16 slots) in both pools, for i < n.
 * Bit-exact. src and dst are int32 device arrays of n block ids in
 * [0, num_blocks); no dst may appear twice or also appear in src.
 *   k_pool, v_pool : [num_blocks, H, 16, D] bf16.  D: 64 or 128.  n <= 65535.
 * Returns ATTN_OK or a negative ATTN_ERR_* code.
 */
int attn_paged_copy_blocks(void* k_pool, void* v_pool, const int32_t* src, const int32_t* dst,
                           int n, int num_blocks, int H, int D, int dtype, void* stream);

/*
 * Host block allocator of the paged cache ([P3] Continuous Batching +
 * PagedAttention: blocks are taken as a sequence grows and returned when it
 * ends; [P4] paged memory management: reference-counted blocks, shared by
 * forked sequences, copied on write; [P1] §3.2 and [P2] §二: requests with a
 * common prefix share its blocks).
 *
 * Pure host bookkeeping, no device memory and no HIP calls. A handle is not
 * thread-safe: one caller at a time. Physical ids run 0 .. num_blocks - 1 and
 * the lowest free id is handed out first on a fresh pool.
 */
typedef struct attn_kv_cache attn_kv_cache;

/* New allocator with every block free and max_seqs empty sequences, each
 * holding at most max_blocks_per_seq blocks. NULL on a non-positive size or
 * out of host memory. */
attn_kv_cache* attn_kv_cache_create(int num_blocks, int max_seqs, int max_blocks_per_seq);

/* Free the handle (NULL is accepted). */
void attn_kv_cache_destroy(attn_kv_cache* cache);

/*
 * Reserve room for n_tokens more tokens of sequence `seq`: new blocks are taken
 * when the last one is full. When the last block is only partly filled and is
 * shared with another sequence (reference count > 1), the sequence gets a
 * private copy: a fresh block replaces it in the table and the pair
 * (shared, fresh) is written to copy_src[0], copy_dst[0] with *n_copies = 1;
 * the caller must copy those blocks on the device (attn_paged_copy_blocks)
 * before writing the new tokens. Otherwise *n_copies = 0.
 * Errors leave the allocator unchanged: ATTN_ERR_NO_BLOCKS when the free
 * blocks do not suffice, ATTN_ERR_BAD_SHAPE for a bad seq, negative n_tokens
 * or a length past max_blocks_per_seq * 16, ATTN_ERR_WORKSPACE when a copy is
 * needed but max_copies < 1 or the copy arrays are NULL.
 */
int attn_kv_cache_append(attn_kv_cache* cache, int seq, int n_tokens, int32_t* copy_src,
                         int32_t* copy_dst, int max_copies, int* n_copies);

/* Make empty sequence `child` share all blocks of `parent` (reference counts
 * +1), with the same length. ATTN_ERR_BAD_SHAPE if child is not empty. */
int attn_kv_cache_fork(attn_kv_cache* cache, int parent, int child);

/* Drop sequence `seq`: its blocks' reference counts go down by one and blocks
 * that reach 0 return to the free pool. The sequence becomes empty. */
int attn_kv_cache_release(attn_kv_cache* cache, int seq);

/* Tokens held by `seq`, or a negative ATTN_ERR_* code. */
int attn_kv_cache_length(const attn_kv_cache* cache, int seq);

/* Number of free blocks, or a negative ATTN_ERR_* code. */
int attn_kv_cache_free_blocks(const attn_kv_cache* cache);

/* Reference count of physical block `block`, or a negative ATTN_ERR_* code. */
int attn_kv_cache_block_refs(const attn_kv_cache* cache, int block);

/* Write the tables to HOST arrays: block_tables [max_seqs, max_blocks_per_seq]
 * int32 (unused entries -1) and seq_lens [max_seqs] int32, ready to copy to the
 * device for the attention and append calls. */
int attn_kv_cache_export(const attn_kv_cache* cache, int32_t* block_tables, int32_t* seq_lens);

/*
 * FP8 KV cache with block-wise scales. The FlashAttention-3 item of [P3] lists
 * FP8 (E4M3 / E5M2) data for the attention products with block-wise
 * quantisation -- each block carries its own scale factor -- and [P2] §五
 * deploys an FP8 KV cache. Here each (physical block, head) of the K pool and
 * of the V pool holds 16 x D E4M3 codes (OCP format: bias 7, max 448, codes
 * 0x7F / 0xFF NaN) and one float32 scale; the stored value is
 * decode(code) * scale. Pools are uint8 [num_blocks, H, 16, D]; scales are
 * float32 [num_blocks, H]. The cache is read at one byte per value, half the
 * bytes of a bf16 cache.
 */

/*
 * attn_paged_append_fp8 -- write n_new new bf16 tokens of K and V into FP8
 * pools (positions as for attn_paged_append). For each (block, head) that
 * receives tokens: s_old is its stored scale, or 0 when the append starts at
 * slot 0 of the block (a fresh block: a stale scale is ignored);
 * s_new = max(s_old, max|new values| / 448); if s_new > s_old the block's
 * earlier slots are re-encoded as e4m3((decode(code) * s_old) / s_new); new
 * values are stored as e4m3(x / s_new) (0 when s_new = 0). Float32 arithmetic,
 * IEEE division, round to nearest even after clamping to +-448. New values
 * must be finite.
 *
 *   k_new, v_new     : [B, H, n_new, D] bf16.
 *   k_pool, v_pool   : [num_blocks, H, 16, D] uint8 (E4M3 codes), in place.
 *   k_scale, v_scale : [num_blocks, H] float32, in place.
 *   block_tables, seq_lens, D, block_size: as for attn_paged_append.
 * Sequences must not share a destination block. Returns ATTN_OK or a negative
 * ATTN_ERR_* code.
 */
int attn_paged_append_fp8(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                          float* k_scale, float* v_scale, const int32_t* block_tables,
                          const int32_t* seq_lens, int B, int H, int n_new, int D,
                          int num_blocks, int max_blocks_per_seq, int block_size, void* stream);

/*
 * attn_paged_copy_blocks_fp8 -- attn_paged_copy_blocks for FP8 pools: copies
 * the codes of block src[i] onto dst[i] in both pools, and its H scales in both
 * scale arrays. Bit-exact.
 */
int attn_paged_copy_blocks_fp8(void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                               const int32_t* src, const int32_t* dst, int n, int num_blocks,
                               int H, int D, void* stream);

/*
 * attn_paged_decode_fp8 -- attn_paged_decode_gqa over FP8 pools: the keys and
 * values are decode(code) * scale of their (block, head). q and o stay bf16;
 * codes are widened to bf16 exactly on chip, the K scale multiplies the
 * block's scores and the V scale its probabilities (float32 accumulation).
 *
 *   q, o             : [B, Hq, q_len, D] bf16.
 *   k_pool, v_pool   : [num_blocks, Hkv, 16, D] uint8 E4M3 codes.
 *   k_scale, v_scale : [num_blocks, Hkv] float32.
 *   workspace        : at least attn_paged_gqa_workspace_bytes(B, Hq, Hkv,
 *                      q_len, D, max_blocks_per_seq, num_splits) bytes.
 *   Every other argument as for attn_paged_decode_gqa (Hq == Hkv is plain
 *   multi-head attention). Returns ATTN_OK or a negative ATTN_ERR_* code.
 */
int attn_paged_decode_fp8(const void* q, const void* k_pool, const void* v_pool,
                          const float* k_scale, const float* v_scale, const int32_t* block_tables,
                          const int32_t* seq_lens, void* o, float* lse, int B, int Hq, int Hkv,
                          int q_len, int D, int num_blocks, int max_blocks_per_seq,
                          int block_size, int causal, float scale, int num_splits,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Human-readable text of a status code (static storage). */
const char* attn_status_string(int status);

/* ATTN_VERSION of the built library. */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_TILED_QK_H */
