// Prefill attention for float32 Q, K, V (the exact-precision path).
//
// Same method as the bf16 kernel -- tiling with the online softmax of [P1]
// §2.2, K/V tiles staged in LDS, running max m and exp-sum l per row, one
// division by l after the last tile -- computed in float32 on the vector ALUs
// with accurate expf, because float32 inputs are held to a 1e-5 bound that
// bf16 matrix-core operands cannot meet.
#include "common.h"

namespace attn {

// One wave per query row, one key per lane. For each 64-key tile a lane forms
// the full dot product of its key with the row's query (read from LDS, the
// same address for all lanes), the wave takes the tile's maximum and sum in
// one reduction each, and the PV sum runs with lanes over the head dimension
// (P broadcast through LDS). Every step is float32 on the vector ALUs, with
// accurate expf. The per-key work has no cross-lane chain, so short sequences
// are latency-light.
namespace {
constexpr int R_WAVES = 4;   // query rows per workgroup
constexpr int R_BN = 64;     // keys per tile (one per lane)

// maximum / sum over the 64 lanes of a wave (butterfly)
__device__ __forceinline__ float lanes_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float lanes_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
}  // namespace

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * R_WAVES) void prefill_f32_rows_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int L, int n_qtiles, float scale) {
  constexpr int KP = D + 4;        // K row pitch in LDS (floats): rows start 4 banks apart
  constexpr int DPL = D / 64;      // head-dimension elements per lane in the PV sum
  __shared__ __attribute__((aligned(16))) float ks[R_BN * KP];
  __shared__ __attribute__((aligned(16))) float vs[R_BN * D];
  __shared__ __attribute__((aligned(16))) float qs[R_WAVES * D];
  __shared__ __attribute__((aligned(16))) float ps[R_WAVES * R_BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int bh = blockIdx.x / n_qtiles;
  const int qt = blockIdx.x % n_qtiles;
  const int q0 = qt * R_WAVES;
  const int row = q0 + wave;
  const size_t head_off = (size_t)bh * L * D;

  for (int i = tid; i < R_WAVES * D; i += 64 * R_WAVES) {
    const int r = q0 + i / D;
    qs[i] = r < L ? q[head_off + (size_t)r * D + i % D] : 0.f;
  }
  const int n_kt = CAUSAL ? (min(q0 + R_WAVES, L) - 1) / R_BN + 1 : (L + R_BN - 1) / R_BN;
  const int last = CAUSAL ? min(row, L - 1) / R_BN : n_kt - 1;  // last tile this row sees

  float m = -INFINITY, l = 0.f;
  float acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.f;

  for (int kt = 0; kt < n_kt; ++kt) {
    __syncthreads();  // the previous tile is no longer read
    constexpr int C4 = D / 4;
    for (int i = tid; i < R_BN * C4; i += 64 * R_WAVES) {
      const int r = i / C4, c = i % C4;
      const int key = kt * R_BN + r;
      const size_t at = head_off + (size_t)key * D + 4 * c;
      const f32x4 kv = key < L ? *reinterpret_cast<const f32x4*>(k + at) : f32x4{0.f, 0.f, 0.f, 0.f};
      const f32x4 vv = key < L ? *reinterpret_cast<const f32x4*>(v + at) : f32x4{0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f32x4*>(ks + r * KP + 4 * c) = kv;
      *reinterpret_cast<f32x4*>(vs + r * D + 4 * c) = vv;
    }
    __syncthreads();
    if (row >= L || kt > last) continue;  // wave-uniform

    // score of key kt * 64 + lane: eight partial sums of D / 8 products each,
    // added as a tree (as accurate as the sixteen-lane butterfly it replaces)
    float part[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) part[t] = 0.f;
#pragma unroll
    for (int c = 0; c < D / 4; ++c) {
      const f32x4 qa = *reinterpret_cast<const f32x4*>(qs + wave * D + 4 * c);
      const f32x4 ka = *reinterpret_cast<const f32x4*>(ks + lane * KP + 4 * c);
      float& pt = part[c % 8];
      pt = __builtin_fmaf(qa[0], ka[0], pt);
      pt = __builtin_fmaf(qa[1], ka[1], pt);
      pt = __builtin_fmaf(qa[2], ka[2], pt);
      pt = __builtin_fmaf(qa[3], ka[3], pt);
    }
    const float dot = ((part[0] + part[1]) + (part[2] + part[3])) + ((part[4] + part[5]) + (part[6] + part[7]));
    const int key = kt * R_BN + lane;
    const bool vis = key < L && (!CAUSAL || key <= row);
    const float s = vis ? dot * scale : -INFINITY;
    const float m_new = fmaxf(m, lanes_max(s));  // finite: key kt * 64 <= row is visible
    const float alpha = m == -INFINITY ? 0.f : expf(m - m_new);
    const float p = vis ? expf(s - m_new) : 0.f;
    l = l * alpha + lanes_sum(p);
    m = m_new;
    ps[wave * R_BN + lane] = p;
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's P is in LDS
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] *= alpha;
#pragma unroll 4
    for (int j4 = 0; j4 < R_BN / 4; ++j4) {
      const f32x4 pj = *reinterpret_cast<const f32x4*>(ps + wave * R_BN + 4 * j4);
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < DPL; ++e)
          acc[e] = __builtin_fmaf(pj[t], vs[(4 * j4 + t) * D + e * 64 + lane], acc[e]);
    }
  }

  if (row < L) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[head_off + (size_t)row * D + e * 64 + lane] = acc[e] * inv;
    if (lse != nullptr && lane == 0) lse[(size_t)bh * L + row] = l > 0.f ? m + logf(l) : -INFINITY;
  }
}

template <int D, bool CAUSAL>
static hipError_t launch_f32(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int H, int L, float scale, hipStream_t stream) {
  const int n_qtiles = (L + R_WAVES - 1) / R_WAVES;
  const long long grid = (long long)B * H * n_qtiles;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_f32_rows_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(64 * R_WAVES), 0,
                     stream, (const float*)q, (const float*)k, (const float*)v, (float*)o, lse, L,
                     n_qtiles, scale);
  return hipGetLastError();
}

// Query rows per workgroup of the float32 prefill kernel (sizes its grid).
int prefill_f32_rows() { return R_WAVES; }

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
