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

// Copy physical block src[i] to dst[i] in both pools (all heads, all slots),
// and, for an FP8 cache, the blocks' H scales of both pools.
__global__ __launch_bounds__(256) void paged_copy_blocks_kernel(void* __restrict__ k_pool,
                                                                void* __restrict__ v_pool,
                                                                float* __restrict__ k_scale,
                                                                float* __restrict__ v_scale,
                                                                const int32_t* __restrict__ src,
                                                                const int32_t* __restrict__ dst,
                                                                long long pieces_per_block, int H) {
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
  if (k_scale != nullptr && blockIdx.x == 0) {
    for (int t = threadIdx.x; t < H; t += 256) {
      k_scale[(size_t)dst[i] * H + t] = k_scale[(size_t)src[i] * H + t];
      v_scale[(size_t)dst[i] * H + t] = v_scale[(size_t)src[i] * H + t];
    }
  }
}

// ---- FP8 (E4M3) cache: codes plus one float32 scale per (block, head)
//
// One wave per (block touched, head, sequence) and per pool. The wave's 64
// lanes cover the block's 16 slots x D values (slot = lane / 4, D/4 values
// each). The scale only grows: s_new = max(s_old, amax(new values) / 448),
// with s_old = 0 when the append starts at slot 0 (a fresh block). If it grew,
// the slots already present are re-encoded as e4m3((decode(code) * s_old) /
// s_new); new values are encoded as e4m3(x / s_new), 0 when s_new is 0. The
// arithmetic is float32 with IEEE division, and the conversion rounds to
// nearest even after clamping to +-448 (the largest E4M3 magnitude).

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}

__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  auto cl = [](float x) { return fminf(fmaxf(x, -448.f), 448.f); };
  uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(a), cl(b), 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(cl(c), cl(d), w, true);
}

template <int D>
__device__ __forceinline__ void append_fp8_pool(const bf16* __restrict__ src_tok, bool is_new,
                                                bool is_old, int s0, uint8_t* __restrict__ slab,
                                                float* __restrict__ scale_ptr, int lane) {
  constexpr int VPL = D / 4;  // values per lane
  float x[VPL];
  float amax = 0.f;
  if (is_new) {
#pragma unroll
    for (int i = 0; i < VPL / 8; ++i) {
      const u32x4 w = reinterpret_cast<const u32x4*>(src_tok)[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[8 * i + 2 * j] = __builtin_bit_cast(float, w[j] << 16);
        x[8 * i + 2 * j + 1] = __builtin_bit_cast(float, w[j] & 0xffff0000u);
      }
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i) amax = fmaxf(amax, fabsf(x[i]));
  }
  amax = wave_max(amax);
  const float s_old = s0 == 0 ? 0.f : *scale_ptr;
  const float s_new = fmaxf(s_old, amax / 448.f);
  u32x4* codes = reinterpret_cast<u32x4*>(slab);  // this lane's VPL code bytes
  if (is_old && s_new > s_old) {
#pragma unroll
    for (int i = 0; i < VPL / 16; ++i) {
      const u32x4 w = codes[i];
      u32x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[j], false);
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[j], true);
        o[j] = e4m3_pack4((lo[0] * s_old) / s_new, (lo[1] * s_old) / s_new,
                          (hi[0] * s_old) / s_new, (hi[1] * s_old) / s_new);
      }
      codes[i] = o;
    }
  }
  if (is_new) {
#pragma unroll
    for (int i = 0; i < VPL / 16; ++i) {
      u32x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float* v4 = x + 16 * i + 4 * j;
        o[j] = s_new > 0.f ? e4m3_pack4(v4[0] / s_new, v4[1] / s_new, v4[2] / s_new, v4[3] / s_new)
                           : 0u;
      }
      codes[i] = o;
    }
  }
  if (lane == 0) *scale_ptr = s_new;
}

template <int D>
__global__ __launch_bounds__(64) void paged_append_fp8_kernel(
    const bf16* __restrict__ k_new, const bf16* __restrict__ v_new, uint8_t* __restrict__ k_pool,
    uint8_t* __restrict__ v_pool, float* __restrict__ k_scale, float* __restrict__ v_scale,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ seq_lens, int H,
    int n_new, int max_blocks) {
  const int lane = threadIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int len = seq_lens[b];
  const int first = max(len - n_new, 0);
  if (first >= len) return;
  const int lb = first / 16 + (int)blockIdx.x;  // logical block of this wave
  if (lb * 16 >= len) return;
  const int s0 = max(first - lb * 16, 0);       // first new slot in the block
  const int s1 = min(len - lb * 16, 16);        // one past the last
  const int phys = block_tables[(size_t)b * max_blocks + lb];
  if (phys < 0) return;
  const int slot = lane >> 2;
  const int d0 = (lane & 3) * (D / 4);
  const bool is_new = slot >= s0 && slot < s1;
  const bool is_old = slot < s0;
  const int t = lb * 16 + slot - (len - n_new);  // new-token index (valid when is_new)
  const size_t tok = (((size_t)b * H + h) * n_new + (is_new ? t : 0)) * D + d0;
  const size_t sidx = (size_t)phys * H + h;
  const size_t slab = (sidx * 16 + slot) * D + d0;
  append_fp8_pool<D>(k_new + tok, is_new, is_old, s0, k_pool + slab, k_scale + sidx, lane);
  append_fp8_pool<D>(v_new + tok, is_new, is_old, s0, v_pool + slab, v_scale + sidx, lane);
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

static hipError_t copy_blocks(void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                              const int32_t* src, const int32_t* dst, int n, int H,
                              long long block_bytes, hipStream_t stream) {
  const long long pieces = block_bytes / 16;  // 16-byte pieces per block
  const long long wgs = (pieces + 255) / 256;
  dim3 grid((unsigned)(wgs < 64 ? wgs : 64), n);
  hipLaunchKernelGGL(paged_copy_blocks_kernel, grid, dim3(256), 0, stream, k_pool, v_pool,
                     k_scale, v_scale, src, dst, pieces, H);
  return hipGetLastError();
}

hipError_t launch_paged_copy_blocks(void* k_pool, void* v_pool, const int32_t* src,
                                    const int32_t* dst, int n, int H, int D, hipStream_t stream) {
  return copy_blocks(k_pool, v_pool, nullptr, nullptr, src, dst, n, H, (long long)H * 16 * D * 2,
                     stream);
}

hipError_t launch_paged_copy_blocks_fp8(void* k_pool, void* v_pool, float* k_scale,
                                        float* v_scale, const int32_t* src, const int32_t* dst,
                                        int n, int H, int D, hipStream_t stream) {
  return copy_blocks(k_pool, v_pool, k_scale, v_scale, src, dst, n, H, (long long)H * 16 * D,
                     stream);
}

hipError_t launch_paged_append_fp8(const void* k_new, const void* v_new, void* k_pool,
                                   void* v_pool, float* k_scale, float* v_scale,
                                   const int32_t* block_tables, const int32_t* seq_lens, int B,
                                   int H, int n_new, int D, int max_blocks, hipStream_t stream) {
  // logical blocks touched per sequence: at most ceil(n_new / 16) + 1
  dim3 grid((unsigned)(n_new / 16 + 2), H, B);
  if (D == 128)
    hipLaunchKernelGGL(paged_append_fp8_kernel<128>, grid, dim3(64), 0, stream,
                       (const bf16*)k_new, (const bf16*)v_new, (uint8_t*)k_pool, (uint8_t*)v_pool,
                       k_scale, v_scale, block_tables, seq_lens, H, n_new, max_blocks);
  else
    hipLaunchKernelGGL(paged_append_fp8_kernel<64>, grid, dim3(64), 0, stream,
                       (const bf16*)k_new, (const bf16*)v_new, (uint8_t*)k_pool, (uint8_t*)v_pool,
                       k_scale, v_scale, block_tables, seq_lens, H, n_new, max_blocks);
  return hipGetLastError();
}

}  // namespace attn
