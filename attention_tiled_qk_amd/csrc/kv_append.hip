// Writing new tokens into the paged KV cache, and whole-block copies.
//
// What is computed: token t of the n_new tokens of sequence b -- absolute
// position p = seq_lens[b] - n_new + t -- is stored in physical block
// block_tables[b][p / 16], slot p % 16, of the K and V pools: the inverse of
// the gather that attention performs through the same table ([P1] §3.2; the
// Continuous Batching + PagedAttention item of [P3]: blocks are filled as
// tokens arrive). Block copies serve copy-on-write of a shared block before a
// sequence writes into it ([P4], the fanzheng.org survey's subsection on paged
// memory management: reference-counted blocks shared between sequences).
//
// Both kernels are plain 16-byte-per-lane copies: one lane per 16 bytes of a
// token's row, rows of one (sequence, head) in consecutive lanes, so that each
// wave reads and writes contiguous runs of the source and destination.
#include "common.h"

namespace attn {

template <int D>
__global__ __launch_bounds__(256) void paged_append_kernel(const bf16* __restrict__ k_new,
                                                           const bf16* __restrict__ v_new,
                                                           bf16* __restrict__ k_pool,
                                                           bf16* __restrict__ v_pool,
                                                           const int32_t* __restrict__ block_tables,
                                                           const int32_t* __restrict__ seq_lens,
                                                           int H, int n_new, int max_blocks) {
  constexpr int CPR = D / 8;  // 16-byte pieces per row
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const long long piece = (long long)blockIdx.x * 256 + threadIdx.x;
  const int t = (int)(piece / CPR);
  const int c = (int)(piece % CPR);
  if (t >= n_new) return;
  const int pos = seq_lens[b] - n_new + t;
  if (pos < 0) return;  // a sequence shorter than the new tokens: nothing to place
  const int phys = block_tables[(size_t)b * max_blocks + (pos >> 4)];
  if (phys < 0) return;
  const size_t dst = (((size_t)phys * H + h) * 16 + (pos & 15)) * D + c * 8;
  const size_t src = (((size_t)b * H + h) * n_new + t) * D + c * 8;
  *reinterpret_cast<u32x4*>(k_pool + dst) = *reinterpret_cast<const u32x4*>(k_new + src);
  *reinterpret_cast<u32x4*>(v_pool + dst) = *reinterpret_cast<const u32x4*>(v_new + src);
}

// Copy physical block src[i] to dst[i] in both pools (all heads, all slots).
__global__ __launch_bounds__(256) void paged_copy_blocks_kernel(bf16* __restrict__ k_pool,
                                                                bf16* __restrict__ v_pool,
                                                                const int32_t* __restrict__ src,
                                                                const int32_t* __restrict__ dst,
                                                                long long pieces_per_block) {
  const int i = blockIdx.y;
  const size_t from = (size_t)src[i] * pieces_per_block;
  const size_t to = (size_t)dst[i] * pieces_per_block;
  u32x4* kp = reinterpret_cast<u32x4*>(k_pool);
  u32x4* vp = reinterpret_cast<u32x4*>(v_pool);
  for (long long p = (long long)blockIdx.x * 256 + threadIdx.x; p < pieces_per_block;
       p += (long long)gridDim.x * 256) {
    kp[to + p] = kp[from + p];
    vp[to + p] = vp[from + p];
  }
}

hipError_t launch_paged_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                               const int32_t* block_tables, const int32_t* seq_lens, int B, int H,
                               int n_new, int D, int max_blocks, hipStream_t stream) {
  const long long pieces = (long long)n_new * (D / 8);
  dim3 grid((unsigned)((pieces + 255) / 256), H, B);
  if (D == 128)
    hipLaunchKernelGGL(paged_append_kernel<128>, grid, dim3(256), 0, stream, (const bf16*)k_new,
                       (const bf16*)v_new, (bf16*)k_pool, (bf16*)v_pool, block_tables, seq_lens, H,
                       n_new, max_blocks);
  else
    hipLaunchKernelGGL(paged_append_kernel<64>, grid, dim3(256), 0, stream, (const bf16*)k_new,
                       (const bf16*)v_new, (bf16*)k_pool, (bf16*)v_pool, block_tables, seq_lens, H,
                       n_new, max_blocks);
  return hipGetLastError();
}

hipError_t launch_paged_copy_blocks(void* k_pool, void* v_pool, const int32_t* src,
                                    const int32_t* dst, int n, int H, int D, hipStream_t stream) {
  const long long pieces = (long long)H * 16 * D / 8;  // 16-byte pieces per block
  const long long wgs = (pieces + 255) / 256;
  dim3 grid((unsigned)(wgs < 64 ? wgs : 64), n);
  hipLaunchKernelGGL(paged_copy_blocks_kernel, grid, dim3(256), 0, stream, (bf16*)k_pool,
                     (bf16*)v_pool, src, dst, pieces);
  return hipGetLastError();
}

}  // namespace attn
