// Prefill attention for float32 Q, K, V (the exact-precision path).
//
// Same method as the bf16 kernel -- tiling with the online softmax of [P1]
// §2.2, K/V tiles staged in LDS, running max m and exp-sum l per row, one
// division by l after the last tile -- computed in float32 on the vector ALUs
// with accurate expf, because float32 inputs are held to a 1e-5 bound that
// bf16 matrix-core operands cannot meet. Each query row is owned by sixteen
// lanes (a sixteenth of the head dimension each, partial dot products summed
// by a shuffle tree); a workgroup covers 8 rows and walks 32- or 64-key tiles, so
// even a short sequence spreads over several CUs. Tiles arrive with 16-byte
// loads into registers one tile ahead: the loads of tile j+1 are in flight
// while tile j is computed, and reach LDS after the next barrier.
#include "common.h"

namespace attn {

namespace {
constexpr int F_LPR = 16;            // lanes per query row
constexpr int F_BM = 128 / F_LPR;    // query rows per workgroup (128 threads)
// keys per tile: 64 at D = 64 (fewer barriers and load round trips), 32 at
// D = 128, where the registers staging a 64-key tile would not fit
constexpr int f32_tile_keys(int D) { return D == 64 ? 64 : 32; }
}  // namespace

template <int D, bool CAUSAL>
__global__ __launch_bounds__(128) void prefill_f32_kernel(const float* __restrict__ q,
                                                          const float* __restrict__ k,
                                                          const float* __restrict__ v,
                                                          float* __restrict__ o,
                                                          float* __restrict__ lse, int L,
                                                          int n_qtiles, float scale) {
  constexpr int F_BN = f32_tile_keys(D);
  constexpr int HD = D / F_LPR;
  constexpr int PITCH = D + 4;
  __shared__ __attribute__((aligned(16))) float ks[F_BN * PITCH];
  __shared__ __attribute__((aligned(16))) float vs[F_BN * PITCH];

  const int tid = threadIdx.x;
  const int slice = tid % F_LPR;  // which slice of the head dimension this lane holds
  const int bh = blockIdx.x / n_qtiles;
  const int qt = blockIdx.x % n_qtiles;
  const int row = qt * F_BM + tid / F_LPR;
  const size_t head_off = (size_t)bh * L * D;

  float qr[HD], acc[HD];
#pragma unroll
  for (int d = 0; d < HD; ++d) {
    qr[d] = row < L ? q[head_off + (size_t)row * D + slice * HD + d] : 0.f;
    acc[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  const int n_all = (L + F_BN - 1) / F_BN;
  const int n_kt = CAUSAL ? min(n_all, (min(qt * F_BM + F_BM, L) - 1) / F_BN + 1) : n_all;

  // 16-byte piece u of this thread: tile row (tid + 128 u) / (D / 4), column
  // 4 ((tid + 128 u) % (D / 4)); keys past L read as zeros
  constexpr int C4 = D / 4;
  constexpr int VEC = F_BN * C4 / 128;
  f32x4 kreg[VEC], vreg[VEC];
  auto fetch = [&](int kt) {
#pragma unroll
    for (int u = 0; u < VEC; ++u) {
      const int i4 = tid + 128 * u;
      const int key = kt * F_BN + i4 / C4;
      const size_t at = head_off + (size_t)key * D + 4 * (i4 % C4);
      kreg[u] = key < L ? *reinterpret_cast<const f32x4*>(k + at) : f32x4{0.f, 0.f, 0.f, 0.f};
      vreg[u] = key < L ? *reinterpret_cast<const f32x4*>(v + at) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  fetch(0);

  for (int kt = 0; kt < n_kt; ++kt) {
    __syncthreads();  // every lane is done reading the previous tile
#pragma unroll
    for (int u = 0; u < VEC; ++u) {
      const int i4 = tid + 128 * u;
      const int at = (i4 / C4) * PITCH + 4 * (i4 % C4);
      *reinterpret_cast<f32x4*>(ks + at) = kreg[u];
      *reinterpret_cast<f32x4*>(vs + at) = vreg[u];
    }
    __syncthreads();
    if (kt + 1 < n_kt) fetch(kt + 1);

    float s[F_BN];
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < F_BN; ++j) {
      float part = 0.f;
#pragma unroll
      for (int d = 0; d < HD; ++d) part = __builtin_fmaf(qr[d], ks[j * PITCH + slice * HD + d], part);
      float full = part;
#pragma unroll
      for (int x = 1; x < F_LPR; x <<= 1) full += __shfl_xor(full, x);
      const int key = kt * F_BN + j;
      const bool vis = key < L && (!CAUSAL || key <= row);
      s[j] = vis ? full * scale : -INFINITY;
      mt = fmaxf(mt, s[j]);
    }
    const float m_new = fmaxf(m, mt);
    if (m_new != -INFINITY) {
      const float alpha = m == -INFINITY ? 0.f : expf(m - m_new);
      l *= alpha;
#pragma unroll
      for (int d = 0; d < HD; ++d) acc[d] *= alpha;
#pragma unroll
      for (int j = 0; j < F_BN; ++j) {
        const float p = s[j] == -INFINITY ? 0.f : expf(s[j] - m_new);
        l += p;
#pragma unroll
        for (int d = 0; d < HD; ++d) acc[d] = __builtin_fmaf(p, vs[j * PITCH + slice * HD + d], acc[d]);
      }
      m = m_new;
    }
  }

  if (row < L) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int d = 0; d < HD; ++d) o[head_off + (size_t)row * D + slice * HD + d] = acc[d] * inv;
    if (lse != nullptr && slice == 0) lse[(size_t)bh * L + row] = l > 0.f ? m + logf(l) : -INFINITY;
  }
}

template <int D, bool CAUSAL>
static hipError_t launch_f32(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int H, int L, float scale, hipStream_t stream) {
  const int n_qtiles = (L + F_BM - 1) / F_BM;
  const long long grid = (long long)B * H * n_qtiles;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_f32_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(128), 0, stream,
                     (const float*)q, (const float*)k, (const float*)v, (float*)o, lse, L,
                     n_qtiles, scale);
  return hipGetLastError();
}

hipError_t launch_prefill_f32(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int H, int L, int D, int causal, float scale,
                              hipStream_t stream) {
  if (D == 128)
    return causal ? launch_f32<128, true>(q, k, v, o, lse, B, H, L, scale, stream)
                  : launch_f32<128, false>(q, k, v, o, lse, B, H, L, scale, stream);
  return causal ? launch_f32<64, true>(q, k, v, o, lse, B, H, L, scale, stream)
                : launch_f32<64, false>(q, k, v, o, lse, B, H, L, scale, stream);
}

}  // namespace attn
