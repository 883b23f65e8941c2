// Host side of the C ABI declared in include/attn.h: argument validation, the
// split-count choice for paged decode, and kernel launches on the caller's
// stream. Everything is checked before anything is enqueued; the library owns
// no memory besides the per-GPU scratch array of the no-allocation decode
// entry point, and keeps no state besides per-kernel launch attributes and
// that array's device addresses.
#include <cmath>
#include <cstdint>
#include <limits>
#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/attn.h"

namespace attn {
hipError_t launch_prefill_bf16(const void*, const void*, const void*, void*, float*, int, int, int,
                               int, int, float, hipStream_t);
hipError_t launch_paged_prefill_bf16(const void*, const void*, const void*, const int32_t*,
                                     const int32_t*, void*, float*, int, int, int, int, int, int,
                                     float, hipStream_t, const int32_t*, int, int);
int paged_prefill_max_blocks();
hipError_t launch_prefill_f32(const void*, const void*, const void*, void*, float*, int, int, int,
                              int, int, float, hipStream_t);
hipError_t launch_paged_attn(const void*, const void*, const void*, const float*, const float*,
                             const int32_t*,
                             const int32_t*, void*, float*, float*, float*, int, int, int, int, int,
                             int, int, int, float, hipStream_t);
hipError_t launch_lse_merge(const float*, const float*, void*, float*, long long, int, int, int,
                            hipStream_t);
hipError_t launch_paged_gather(const void*, const int32_t*, const int32_t*, void*, int, int, int,
                               int, int, hipStream_t);
hipError_t launch_paged_append(const void*, const void*, void*, void*, const int32_t*,
                               const int32_t*, int, int, int, int, int, hipStream_t);
hipError_t launch_paged_copy_blocks(void*, void*, const int32_t*, const int32_t*, int, int, int,
                                    hipStream_t);
hipError_t launch_paged_append_fp8(const void*, const void*, void*, void*, float*, float*,
                                   const int32_t*, const int32_t*, int, int, int, int, int,
                                   hipStream_t);
hipError_t launch_paged_copy_blocks_fp8(void*, void*, float*, float*, const int32_t*,
                                        const int32_t*, int, int, int, hipStream_t);
hipError_t launch_check_tables(const int32_t*, const int32_t*, int, int, int, int, int32_t*,
                               hipStream_t);
hipError_t launch_check_append(const int32_t*, const int32_t*, int, int, int, int, int32_t*,
                               hipStream_t);
hipError_t launch_check_ragged(const int32_t*, const int32_t*, int, int, int, int32_t*,
                               hipStream_t);
hipError_t launch_check_ids(const int32_t*, const int32_t*, int, int, int32_t*, hipStream_t);
int prefill_bf16_rows();
int prefill_f32_rows();
}  // namespace attn

namespace {

constexpr long long kMaxGrid = 0x7fffffffLL;
// work-items of a one-dimensional launch (grid x block) must fit 32 bits
constexpr long long kMaxItems = 0xffffffffLL;
constexpr int kMaxMergeSplits = 1024;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

// Product of positive ints, or -1 on overflow past 2^62.
long long checked_mul(std::initializer_list<long long> xs) {
  long long r = 1;
  for (long long x : xs) {
    if (x <= 0) return -1;
    if (r > (1LL << 62) / x) return -1;
    r *= x;
  }
  return r;
}

// Split count for paged decode when the caller leaves it to the library:
// splits of about `per` blocks on the longest possible sequence, raised
// towards enough (split, head, sequence) items to cover the chip several times
// as long as every split keeps at least 4 blocks.
// * Batches of up to 64 sequences run longest sequence first in the kernel,
//   which evens the end of the launch when the splits are long; they take
//   splits of about 128 blocks (64 sequences x 40 heads, 128 to 4096 keys: 2
//   splits 413 us, 8 splits 430 us).
// * Larger batches keep the batch order and splits of about 32 blocks (512
//   tokens), so that items carry similar amounts of work whatever the length
//   mix.
// * Grouped-query items write `group` partial rows per split and serve `group`
//   heads from one read; they take splits of about 256 blocks and a quarter of
//   the covering target: such launches have few items, which then run four
//   waves each (merged in LDS) (64 sequences, 8 KV heads, group 8: 1 split
//   91.7 us, 2 splits 95-97 us, 4 splits in batch order 109 us).
int auto_splits(int B, int H, int max_blocks, int group) {
  const long long per = group > 1 ? 256 : B <= 64 ? 128 : 32;
  long long s = ((long long)max_blocks + per - 1) / per;
  const long long waves = (long long)B * H;
  long long fill = ((group > 1 ? 512 : 2048) + waves - 1) / waves;
  if (fill > max_blocks / 4) fill = max_blocks / 4;
  if (s < fill) s = fill;
  if (s < 1) s = 1;
  if (s > ATTN_PAGED_MAX_SPLITS) s = ATTN_PAGED_MAX_SPLITS;
  return (int)s;
}

size_t workspace_for(int B, int H, int q_len, int D, int S) {
  if (S <= 1) return 0;
  const long long rows = checked_mul({B, H, q_len, S});
  if (rows < 0) return 0;
  return (size_t)rows * (size_t)(D + 1) * sizeof(float);
}

}  // namespace

extern "C" {

int attn_version(void) { return ATTN_VERSION; }

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL_PTR: return "a required pointer is NULL";
    case ATTN_ERR_BAD_SHAPE: return "a size is non-positive or the shapes disagree";
    case ATTN_ERR_BAD_DTYPE: return "dtype not supported by this entry point";
    case ATTN_ERR_UNSUPPORTED: return "head_dim, q_len, block_size or split count is outside the supported set";
    case ATTN_ERR_MISALIGNED: return "a pointer is not 16-byte aligned";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_OVERFLOW: return "sizes overflow the kernels' indexing";
    case ATTN_ERR_HIP: return "kernel launch failed";
    case ATTN_ERR_NO_BLOCKS: return "the block pool has too few free blocks";
    case ATTN_ERR_SCRATCH: return "split-KV partials exceed the static scratch (ATTN_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int attn_prefill(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int L, int D, int causal, float scale, int dtype, void* stream) {
  if (!q || !k || !v || !o) return ATTN_ERR_NULL_PTR;
  if (B <= 0 || H <= 0 || L <= 0) return ATTN_ERR_BAD_SHAPE;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_BAD_DTYPE;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if (causal != 0 && causal != 1) return ATTN_ERR_BAD_SHAPE;
  if (!std::isfinite(scale)) return ATTN_ERR_BAD_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_ERR_MISALIGNED;
  if (lse && !aligned4(lse)) return ATTN_ERR_MISALIGNED;
  if (checked_mul({B, H, L, D, 4}) < 0) return ATTN_ERR_OVERFLOW;
  // the bf16 kernel addresses one head's K/V through a 32-bit byte range
  if ((long long)L * D * 2 > 0x7fffffffLL) return ATTN_ERR_OVERFLOW;
  const int rows = dtype == ATTN_BF16 ? attn::prefill_bf16_rows() : attn::prefill_f32_rows();
  if ((long long)B * H * ((L + rows - 1) / rows) > kMaxGrid) return ATTN_ERR_OVERFLOW;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dtype == ATTN_BF16)
    return hip_status(attn::launch_prefill_bf16(q, k, v, o, lse, B, H, L, D, causal, scale, s));
  return hip_status(attn::launch_prefill_f32(q, k, v, o, lse, B, H, L, D, causal, scale, s));
}

}  // extern "C"

namespace {

// Split count the library uses for `Hkv` KV heads (one wave group per split, KV
// head and sequence) when the caller passes num_splits = 0.
int splits_for(int B, int Hkv, int group, int max_blocks_per_seq, int num_splits) {
  return num_splits == 0 ? auto_splits(B, Hkv, max_blocks_per_seq, group) : num_splits;
}

size_t paged_workspace(int B, int Hq, int Hkv, int q_len, int D, int max_blocks_per_seq,
                       int num_splits) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || q_len <= 0 || Hq % Hkv != 0) return 0;
  if ((long long)(Hq / Hkv) * q_len > ATTN_PAGED_MAX_QLEN) return 0;
  if (D != 64 && D != 128) return 0;
  if (max_blocks_per_seq <= 0 || num_splits < 0 || num_splits > ATTN_PAGED_MAX_SPLITS) return 0;
  return workspace_for(B, Hq, q_len, D,
                       splits_for(B, Hkv, Hq / Hkv, max_blocks_per_seq, num_splits));
}

// k_scale == nullptr: bf16 pools; otherwise E4M3 pools (one byte per value)
// with per-(block, head) scales.
int paged_decode(const void* q, const void* k_pool, const void* v_pool, const float* k_scale,
                 const float* v_scale,
                 const int32_t* block_tables, const int32_t* seq_lens, void* o, float* lse, int B,
                 int Hq, int Hkv, int q_len, int D, int num_blocks, int max_blocks_per_seq,
                 int block_size, int causal, float scale, int num_splits, void* workspace,
                 size_t workspace_bytes, int dtype, void* stream) {
  if (!q || !k_pool || !v_pool || !block_tables || !seq_lens || !o) return ATTN_ERR_NULL_PTR;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || q_len <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0)
    return ATTN_ERR_BAD_SHAPE;
  if (Hq % Hkv != 0) return ATTN_ERR_BAD_SHAPE;
  if (dtype != ATTN_BF16) return ATTN_ERR_BAD_DTYPE;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if (block_size != ATTN_BLOCK_SIZE) return ATTN_ERR_UNSUPPORTED;
  const int group = Hq / Hkv;
  if ((long long)group * q_len > ATTN_PAGED_MAX_QLEN) return ATTN_ERR_UNSUPPORTED;
  if (num_splits < 0 || num_splits > ATTN_PAGED_MAX_SPLITS) return ATTN_ERR_UNSUPPORTED;
  if (causal != 0 && causal != 1) return ATTN_ERR_BAD_SHAPE;
  if (!std::isfinite(scale)) return ATTN_ERR_BAD_SHAPE;
  if (Hkv > 65535 || B > 65535) return ATTN_ERR_OVERFLOW;
  if (checked_mul({num_blocks, Hkv, 16, D, k_scale ? 1 : 2}) < 0 ||
      checked_mul({B, max_blocks_per_seq}) < 0 || checked_mul({B, Hq, q_len, D, 2}) < 0 ||
      (long long)max_blocks_per_seq * 16 > 0x7fffffffLL)
    return ATTN_ERR_OVERFLOW;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(o))
    return ATTN_ERR_MISALIGNED;
  if (!aligned4(block_tables) || !aligned4(seq_lens) || (lse && !aligned4(lse)))
    return ATTN_ERR_MISALIGNED;
  if (k_scale && (!aligned4(k_scale) || !aligned4(v_scale))) return ATTN_ERR_MISALIGNED;
  int S = splits_for(B, Hkv, group, max_blocks_per_seq, num_splits);
  // The fp8 kernel runs four waves per (split, head, sequence), merged in LDS
  // (it holds three waves per SIMD, so a workgroup of four does not hold a CU
  // idle behind its slowest wave), and reads half the bytes per block: an
  // eighth of the automatic split count keeps its items long enough for the
  // longest-first order (64 sequences x 40 heads of 128 to 4096 keys: 1 split
  // longest-first 217 us, 2 splits 227 us, 2 splits in batch order 232 us).
  // The workspace size query stays that of the bf16 call, which is never
  // smaller.
  if (k_scale != nullptr && num_splits == 0) S = (S + 7) / 8;
  // the merge runs one workgroup of D threads per (sequence, head, query) row
  if (S > 1 && (long long)B * Hq * q_len * D > kMaxItems) return ATTN_ERR_OVERFLOW;
  const size_t need = workspace_for(B, Hq, q_len, D, S);
  float* o_part = nullptr;
  float* lse_part = nullptr;
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    if (!aligned16(workspace)) return ATTN_ERR_MISALIGNED;
    o_part = static_cast<float*>(workspace);
    lse_part = o_part + (size_t)B * Hq * q_len * S * D;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = attn::launch_paged_attn(q, k_pool, v_pool, k_scale, v_scale, block_tables,
                                         seq_lens, o, lse, o_part,
                                         lse_part, B, Hkv, group, q_len, D, max_blocks_per_seq, S,
                                         causal, scale, s);
  if (e != hipSuccess || S == 1) return hip_status(e);
  return hip_status(attn::launch_lse_merge(o_part, lse_part, o, lse, (long long)B * Hq * q_len, S,
                                           D, 1, s));
}

}  // namespace

extern "C" {

size_t attn_paged_workspace_bytes(int B, int H, int q_len, int D, int max_blocks_per_seq,
                                  int num_splits) {
  return paged_workspace(B, H, H, q_len, D, max_blocks_per_seq, num_splits);
}

int attn_paged_prefill(const void* q, const void* k_pool, const void* v_pool,
                       const int32_t* block_tables, const int32_t* seq_lens, void* o, float* lse,
                       int B, int H, int q_len, int D, int num_blocks, int max_blocks_per_seq,
                       int block_size, int causal, float scale, int dtype, void* stream) {
  if (!q || !k_pool || !v_pool || !block_tables || !seq_lens || !o) return ATTN_ERR_NULL_PTR;
  if (B <= 0 || H <= 0 || q_len <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0)
    return ATTN_ERR_BAD_SHAPE;
  if (dtype != ATTN_BF16) return ATTN_ERR_BAD_DTYPE;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if (block_size != ATTN_BLOCK_SIZE) return ATTN_ERR_UNSUPPORTED;
  if (max_blocks_per_seq > attn::paged_prefill_max_blocks()) return ATTN_ERR_UNSUPPORTED;
  if ((long long)q_len > (long long)max_blocks_per_seq * 16) return ATTN_ERR_BAD_SHAPE;
  if (causal != 0 && causal != 1) return ATTN_ERR_BAD_SHAPE;
  if (!std::isfinite(scale)) return ATTN_ERR_BAD_SHAPE;
  if (checked_mul({num_blocks, H, 16, D, 2}) < 0 || checked_mul({B, max_blocks_per_seq}) < 0 ||
      checked_mul({B, H, q_len, D, 4}) < 0)
    return ATTN_ERR_OVERFLOW;
  const int rows = attn::prefill_bf16_rows();
  if ((long long)B * H * ((q_len + rows - 1) / rows) > kMaxGrid) return ATTN_ERR_OVERFLOW;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(o))
    return ATTN_ERR_MISALIGNED;
  if (!aligned4(block_tables) || !aligned4(seq_lens) || (lse && !aligned4(lse)))
    return ATTN_ERR_MISALIGNED;
  return hip_status(attn::launch_paged_prefill_bf16(q, k_pool, v_pool, block_tables, seq_lens, o,
                                                    lse, B, H, q_len, D, max_blocks_per_seq,
                                                    causal, scale,
                                                    reinterpret_cast<hipStream_t>(stream), nullptr,
                                                    H, num_blocks));
}

int attn_paged_prefill_varlen(const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* block_tables, const int32_t* seq_lens,
                              const int32_t* cu_q_lens, void* o, float* lse, int B, int H,
                              int total_q, int max_q_len, int D, int num_blocks,
                              int max_blocks_per_seq, int block_size, int causal, float scale,
                              int dtype, void* stream) {
  return attn_paged_prefill_gqa(q, k_pool, v_pool, block_tables, seq_lens, cu_q_lens, o, lse, B,
                                H, H, total_q, max_q_len, D, num_blocks, max_blocks_per_seq,
                                block_size, causal, scale, dtype, stream);
}

int attn_paged_prefill_gqa(const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* block_tables, const int32_t* seq_lens,
                           const int32_t* cu_q_lens, void* o, float* lse, int B, int H, int Hkv,
                           int total_q, int max_q_len, int D, int num_blocks,
                           int max_blocks_per_seq, int block_size, int causal, float scale,
                           int dtype, void* stream) {
  if (!q || !k_pool || !v_pool || !block_tables || !seq_lens || !cu_q_lens || !o)
    return ATTN_ERR_NULL_PTR;
  if (B <= 0 || H <= 0 || Hkv <= 0 || total_q <= 0 || max_q_len <= 0 || num_blocks <= 0 ||
      max_blocks_per_seq <= 0)
    return ATTN_ERR_BAD_SHAPE;
  if (H % Hkv != 0) return ATTN_ERR_BAD_SHAPE;
  if (max_q_len > total_q) return ATTN_ERR_BAD_SHAPE;
  if (dtype != ATTN_BF16) return ATTN_ERR_BAD_DTYPE;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if (block_size != ATTN_BLOCK_SIZE) return ATTN_ERR_UNSUPPORTED;
  if (max_blocks_per_seq > attn::paged_prefill_max_blocks()) return ATTN_ERR_UNSUPPORTED;
  if ((long long)max_q_len > (long long)max_blocks_per_seq * 16) return ATTN_ERR_BAD_SHAPE;
  if (causal != 0 && causal != 1) return ATTN_ERR_BAD_SHAPE;
  if (!std::isfinite(scale)) return ATTN_ERR_BAD_SHAPE;
  if (checked_mul({num_blocks, Hkv, 16, D, 2}) < 0 || checked_mul({B, max_blocks_per_seq}) < 0 ||
      checked_mul({total_q, H, D, 4}) < 0)
    return ATTN_ERR_OVERFLOW;
  const int rows = attn::prefill_bf16_rows();
  if ((long long)B * H * ((max_q_len + rows - 1) / rows) > kMaxGrid) return ATTN_ERR_OVERFLOW;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(o))
    return ATTN_ERR_MISALIGNED;
  if (!aligned4(block_tables) || !aligned4(seq_lens) || !aligned4(cu_q_lens) ||
      (lse && !aligned4(lse)))
    return ATTN_ERR_MISALIGNED;
  return hip_status(attn::launch_paged_prefill_bf16(q, k_pool, v_pool, block_tables, seq_lens, o,
                                                    lse, B, H, max_q_len, D, max_blocks_per_seq,
                                                    causal, scale,
                                                    reinterpret_cast<hipStream_t>(stream),
                                                    cu_q_lens, Hkv, num_blocks));
}

size_t attn_paged_gqa_workspace_bytes(int B, int Hq, int Hkv, int q_len, int D,
                                      int max_blocks_per_seq, int num_splits) {
  return paged_workspace(B, Hq, Hkv, q_len, D, max_blocks_per_seq, num_splits);
}

int attn_paged_decode(const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_tables, const int32_t* seq_lens, void* o, float* lse,
                      int B, int H, int q_len, int D, int num_blocks, int max_blocks_per_seq,
                      int block_size, int causal, float scale, int num_splits, void* workspace,
                      size_t workspace_bytes, int dtype, void* stream) {
  return paged_decode(q, k_pool, v_pool, nullptr, nullptr, block_tables, seq_lens, o, lse, B, H,
                      H, q_len, D,
                      num_blocks, max_blocks_per_seq, block_size, causal, scale, num_splits,
                      workspace, workspace_bytes, dtype, stream);
}

int attn_paged_decode_gqa(const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* block_tables, const int32_t* seq_lens, void* o, float* lse,
                          int B, int Hq, int Hkv, int q_len, int D, int num_blocks,
                          int max_blocks_per_seq, int block_size, int causal, float scale,
                          int num_splits, void* workspace, size_t workspace_bytes, int dtype,
                          void* stream) {
  return paged_decode(q, k_pool, v_pool, nullptr, nullptr, block_tables, seq_lens, o, lse, B, Hq,
                      Hkv, q_len, D,
                      num_blocks, max_blocks_per_seq, block_size, causal, scale, num_splits,
                      workspace, workspace_bytes, dtype, stream);
}

}  // extern "C"

// Split-KV partials of attn_paged_decode_noalloc. Each GPU the code object is
// loaded onto holds its own copy until the process ends. Host code never uses
// this name as an address (on the host it only identifies the symbol): the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_addr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of the current device's scratch (looked up on the first call
// on that device, which is current then; the result, or the failure, is kept).
int device_scratch(void** addr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_HIP;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_addr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess || g_scratch_addr[dev] == nullptr) return ATTN_ERR_HIP;
  *addr = g_scratch_addr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_paged_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* block_tables, const int32_t* seq_lens, void* o,
                              float* lse, int B, int Hq, int Hkv, int q_len, int D,
                              int num_blocks, int max_blocks_per_seq, int block_size, int causal,
                              float scale, int num_splits, int dtype, void* stream) {
  if (!q || !k_pool || !v_pool || !block_tables || !seq_lens || !o) return ATTN_ERR_NULL_PTR;
  // 0 for invalid arguments too: paged_decode reports those
  const size_t need = paged_workspace(B, Hq, Hkv, q_len, D, max_blocks_per_seq, num_splits);
  if (need > ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    const int st = device_scratch(&ws);
    if (st != ATTN_OK) return st;
  }
  return paged_decode(q, k_pool, v_pool, nullptr, nullptr, block_tables, seq_lens, o, lse, B, Hq,
                      Hkv, q_len, D, num_blocks, max_blocks_per_seq, block_size, causal, scale,
                      num_splits, ws, need, dtype, stream);
}

int attn_lse_merge(const float* o_part, const float* lse_part, void* o, float* lse, int B, int H,
                   int q_len, int S, int D, int dtype, void* stream) {
  if (!o_part || !lse_part || !o) return ATTN_ERR_NULL_PTR;
  if (B <= 0 || H <= 0 || q_len <= 0 || S <= 0) return ATTN_ERR_BAD_SHAPE;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_BAD_DTYPE;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if (S > kMaxMergeSplits) return ATTN_ERR_UNSUPPORTED;
  const long long rows = checked_mul({B, H, q_len});
  if (rows < 0 || rows > kMaxGrid || rows * D > kMaxItems || checked_mul({rows, S, D, 4}) < 0)
    return ATTN_ERR_OVERFLOW;
  if (!aligned16(o_part) || !aligned16(o)) return ATTN_ERR_MISALIGNED;
  if (!aligned4(lse_part) || (lse && !aligned4(lse))) return ATTN_ERR_MISALIGNED;
  return hip_status(attn::launch_lse_merge(o_part, lse_part, o, lse, rows, S, D,
                                           dtype == ATTN_BF16 ? 1 : 0,
                                           reinterpret_cast<hipStream_t>(stream)));
}

int attn_paged_gather(const void* pool, const int32_t* block_tables, const int32_t* seq_lens,
                      void* out, int B, int H, int D, int num_blocks, int max_blocks_per_seq,
                      int max_seq_len, void* stream) {
  if (!pool || !block_tables || !seq_lens || !out) return ATTN_ERR_NULL_PTR;
  if (B <= 0 || H <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 || max_seq_len <= 0)
    return ATTN_ERR_BAD_SHAPE;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if (H > 65535 || B > 65535) return ATTN_ERR_OVERFLOW;
  if (checked_mul({B, H, max_seq_len, D, 2}) < 0 || checked_mul({num_blocks, H, 16, D, 2}) < 0)
    return ATTN_ERR_OVERFLOW;
  if (((long long)max_seq_len * (D / 8) + 255) / 256 > kMaxGrid) return ATTN_ERR_OVERFLOW;
  if (!aligned16(pool) || !aligned16(out)) return ATTN_ERR_MISALIGNED;
  if (!aligned4(block_tables) || !aligned4(seq_lens)) return ATTN_ERR_MISALIGNED;
  return hip_status(attn::launch_paged_gather(pool, block_tables, seq_lens, out, B, H, D,
                                              max_blocks_per_seq, max_seq_len,
                                              reinterpret_cast<hipStream_t>(stream)));
}

int attn_paged_check_tables(const int32_t* block_tables, const int32_t* seq_lens, int B,
                            int min_len, int num_blocks, int max_blocks_per_seq, int32_t* bad,
                            void* stream) {
  if (!block_tables || !seq_lens || !bad) return ATTN_ERR_NULL_PTR;
  if (B <= 0 || min_len < 0 || num_blocks <= 0 || max_blocks_per_seq <= 0) return ATTN_ERR_BAD_SHAPE;
  if (checked_mul({B, max_blocks_per_seq}) < 0) return ATTN_ERR_OVERFLOW;
  if (!aligned4(block_tables) || !aligned4(seq_lens) || !aligned4(bad)) return ATTN_ERR_MISALIGNED;
  return hip_status(attn::launch_check_tables(block_tables, seq_lens, B, min_len, num_blocks,
                                              max_blocks_per_seq, bad,
                                              reinterpret_cast<hipStream_t>(stream)));
}

int attn_paged_check_append(const int32_t* block_tables, const int32_t* seq_lens, int B, int n_new,
                            int num_blocks, int max_blocks_per_seq, int32_t* bad, void* stream) {
  if (!block_tables || !seq_lens || !bad) return ATTN_ERR_NULL_PTR;
  if (B <= 0 || n_new <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0) return ATTN_ERR_BAD_SHAPE;
  if (checked_mul({B, max_blocks_per_seq}) < 0) return ATTN_ERR_OVERFLOW;
  if (!aligned4(block_tables) || !aligned4(seq_lens) || !aligned4(bad)) return ATTN_ERR_MISALIGNED;
  return hip_status(attn::launch_check_append(block_tables, seq_lens, B, n_new, num_blocks,
                                              max_blocks_per_seq, bad,
                                              reinterpret_cast<hipStream_t>(stream)));
}

int attn_paged_check_ragged(const int32_t* cu_q_lens, const int32_t* seq_lens, int B, int total_q,
                            int max_q_len, int32_t* bad, void* stream) {
  if (!cu_q_lens || !seq_lens || !bad) return ATTN_ERR_NULL_PTR;
  if (B <= 0 || total_q <= 0 || max_q_len <= 0) return ATTN_ERR_BAD_SHAPE;
  if (!aligned4(cu_q_lens) || !aligned4(seq_lens) || !aligned4(bad)) return ATTN_ERR_MISALIGNED;
  return hip_status(attn::launch_check_ragged(cu_q_lens, seq_lens, B, total_q, max_q_len, bad,
                                              reinterpret_cast<hipStream_t>(stream)));
}

int attn_paged_check_ids(const int32_t* src, const int32_t* dst, int n, int num_blocks,
                         int32_t* bad, void* stream) {
  if (!src || !dst || !bad) return ATTN_ERR_NULL_PTR;
  if (n <= 0 || num_blocks <= 0) return ATTN_ERR_BAD_SHAPE;
  if (!aligned4(src) || !aligned4(dst) || !aligned4(bad)) return ATTN_ERR_MISALIGNED;
  return hip_status(attn::launch_check_ids(src, dst, n, num_blocks, bad,
                                           reinterpret_cast<hipStream_t>(stream)));
}

int attn_paged_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                      const int32_t* block_tables, const int32_t* seq_lens, int B, int H,
                      int n_new, int D, int num_blocks, int max_blocks_per_seq, int block_size,
                      int dtype, void* stream) {
  if (!k_new || !v_new || !k_pool || !v_pool || !block_tables || !seq_lens)
    return ATTN_ERR_NULL_PTR;
  if (B <= 0 || H <= 0 || n_new <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0)
    return ATTN_ERR_BAD_SHAPE;
  if (dtype != ATTN_BF16) return ATTN_ERR_BAD_DTYPE;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if (block_size != ATTN_BLOCK_SIZE) return ATTN_ERR_UNSUPPORTED;
  if ((long long)n_new > (long long)max_blocks_per_seq * 16) return ATTN_ERR_BAD_SHAPE;
  if (H > 65535 || B > 65535) return ATTN_ERR_OVERFLOW;
  if (checked_mul({B, H, n_new, D, 2}) < 0 || checked_mul({num_blocks, H, 16, D, 2}) < 0 ||
      checked_mul({B, max_blocks_per_seq}) < 0)
    return ATTN_ERR_OVERFLOW;
  if (((long long)n_new * (D / 8) + 255) / 256 > kMaxGrid) return ATTN_ERR_OVERFLOW;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool))
    return ATTN_ERR_MISALIGNED;
  if (!aligned4(block_tables) || !aligned4(seq_lens)) return ATTN_ERR_MISALIGNED;
  return hip_status(attn::launch_paged_append(k_new, v_new, k_pool, v_pool, block_tables,
                                              seq_lens, B, H, n_new, D, max_blocks_per_seq,
                                              reinterpret_cast<hipStream_t>(stream)));
}

int attn_paged_copy_blocks(void* k_pool, void* v_pool, const int32_t* src, const int32_t* dst,
                           int n, int num_blocks, int H, int D, int dtype, void* stream) {
  if (!k_pool || !v_pool || !src || !dst) return ATTN_ERR_NULL_PTR;
  if (n <= 0 || num_blocks <= 0 || H <= 0) return ATTN_ERR_BAD_SHAPE;
  if (dtype != ATTN_BF16) return ATTN_ERR_BAD_DTYPE;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if (n > 65535) return ATTN_ERR_OVERFLOW;
  if (checked_mul({num_blocks, H, 16, D, 2}) < 0) return ATTN_ERR_OVERFLOW;
  if (!aligned16(k_pool) || !aligned16(v_pool)) return ATTN_ERR_MISALIGNED;
  if (!aligned4(src) || !aligned4(dst)) return ATTN_ERR_MISALIGNED;
  return hip_status(attn::launch_paged_copy_blocks(k_pool, v_pool, src, dst, n, H, D,
                                                   reinterpret_cast<hipStream_t>(stream)));
}

int attn_paged_decode_fp8(const void* q, const void* k_pool, const void* v_pool,
                          const float* k_scale, const float* v_scale, const int32_t* block_tables,
                          const int32_t* seq_lens, void* o, float* lse, int B, int Hq, int Hkv,
                          int q_len, int D, int num_blocks, int max_blocks_per_seq,
                          int block_size, int causal, float scale, int num_splits,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (!k_scale || !v_scale) return ATTN_ERR_NULL_PTR;
  return paged_decode(q, k_pool, v_pool, k_scale, v_scale, block_tables, seq_lens, o, lse, B, Hq,
                      Hkv, q_len, D, num_blocks, max_blocks_per_seq, block_size, causal, scale,
                      num_splits, workspace, workspace_bytes, ATTN_BF16, stream);
}

int attn_paged_append_fp8(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                          float* k_scale, float* v_scale, const int32_t* block_tables,
                          const int32_t* seq_lens, int B, int H, int n_new, int D,
                          int num_blocks, int max_blocks_per_seq, int block_size, void* stream) {
  if (!k_new || !v_new || !k_pool || !v_pool || !k_scale || !v_scale || !block_tables ||
      !seq_lens)
    return ATTN_ERR_NULL_PTR;
  if (B <= 0 || H <= 0 || n_new <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0)
    return ATTN_ERR_BAD_SHAPE;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if (block_size != ATTN_BLOCK_SIZE) return ATTN_ERR_UNSUPPORTED;
  if ((long long)n_new > (long long)max_blocks_per_seq * 16) return ATTN_ERR_BAD_SHAPE;
  if (H > 65535 || B > 65535) return ATTN_ERR_OVERFLOW;
  if (checked_mul({B, H, n_new, D, 2}) < 0 || checked_mul({num_blocks, H, 16, D}) < 0 ||
      checked_mul({B, max_blocks_per_seq}) < 0)
    return ATTN_ERR_OVERFLOW;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool))
    return ATTN_ERR_MISALIGNED;
  if (!aligned4(k_scale) || !aligned4(v_scale) || !aligned4(block_tables) || !aligned4(seq_lens))
    return ATTN_ERR_MISALIGNED;
  return hip_status(attn::launch_paged_append_fp8(k_new, v_new, k_pool, v_pool, k_scale, v_scale,
                                                  block_tables, seq_lens, B, H, n_new, D,
                                                  max_blocks_per_seq,
                                                  reinterpret_cast<hipStream_t>(stream)));
}

int attn_paged_copy_blocks_fp8(void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                               const int32_t* src, const int32_t* dst, int n, int num_blocks,
                               int H, int D, void* stream) {
  if (!k_pool || !v_pool || !k_scale || !v_scale || !src || !dst) return ATTN_ERR_NULL_PTR;
  if (n <= 0 || num_blocks <= 0 || H <= 0) return ATTN_ERR_BAD_SHAPE;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if (n > 65535) return ATTN_ERR_OVERFLOW;
  if (checked_mul({num_blocks, H, 16, D}) < 0) return ATTN_ERR_OVERFLOW;
  if (!aligned16(k_pool) || !aligned16(v_pool)) return ATTN_ERR_MISALIGNED;
  if (!aligned4(k_scale) || !aligned4(v_scale) || !aligned4(src) || !aligned4(dst))
    return ATTN_ERR_MISALIGNED;
  return hip_status(attn::launch_paged_copy_blocks_fp8(k_pool, v_pool, k_scale, v_scale, src, dst,
                                                       n, H, D,
                                                       reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
