// Causal / full prefill attention for bf16 Q, K, V on gfx950 matrix cores.
//
// What is computed: O = softmax(scale * Q K^T + mask) V per (batch, head)
// ([P2] §一), by the tiled online-softmax method of [P1] §2.2: Q is cut into
// row tiles (one workgroup each, the query-sequence parallelism that the
// FlashAttention-2 item of [P3] adds), K/V into 64-key tiles streamed through
// LDS; every row keeps a running max m and exp-sum l, the output accumulator is
// rescaled only when m grows, and O is divided by l once after the last tile.
// Nothing of size L x L is ever written to memory.
//
// gfx950 mapping (per workgroup of NW waves, BM = 32 * NW query rows):
//   * each wave owns 32 query rows; Q stays in VGPRs as the B operand of
//     S^T = K Q^T (v_mfma_f32_32x32x16_bf16), so every lane's accumulators hold
//     16 keys of ONE query: the row max / row sum is an in-lane reduction plus
//     one permlane32 swap, and the output accumulator O^T keeps one query per
//     lane too, so its rescale is a broadcast multiply;
//   * P^T feeds O^T += V^T P^T straight from the S^T accumulators (converted to
//     bf16 in registers, no LDS round trip); V^T operands come from the
//     row-major V tile in LDS through ds_read_b64_tr_b16 transposing reads;
//   * K/V tiles are double-buffered in LDS with padded row pitches chosen so
//     the 16-byte K reads and the transposing V reads are free of bank conflicts;
//   * causal: key tiles above a wave's last row are skipped, the mask is only
//     evaluated on tiles that cross the diagonal, workgroups are ordered
//     heavy-first within a head and heads are kept on one XCD (xcd_remap).
#include "common.h"

namespace attn {

namespace {

constexpr int BN = 64;  // keys per tile

template <int D, int NW>
struct PrefillCfg {
  static constexpr int BM = 32 * NW;
  static constexpr int KC = D / 16;          // 16-wide k chunks of the QK^T contraction
  static constexpr int DB = D / 32;          // 32-wide output column blocks
  static constexpr int PK = D * 2 + 16;      // K tile row pitch (bytes)
  static constexpr int PV = D * 2 + 64;      // V tile row pitch (bytes)
  static constexpr int K_BYTES = BN * PK;
  static constexpr int V_BYTES = BN * PV;
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int THREADS = NW * 64;
  static constexpr int CHUNKS = BN * D / 8;  // 16-byte chunks per K (or V) tile
  static constexpr int CPT = CHUNKS / THREADS;
  static_assert(CHUNKS % THREADS == 0, "tile chunks must divide evenly");
};

}  // namespace

template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void prefill_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    bf16* __restrict__ o, float* __restrict__ lse, int BH, int L, int n_qtiles, float scale) {
  using C = PrefillCfg<D, NW>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  ATTN_LDS unsigned char* smem = (ATTN_LDS unsigned char*)smem_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;  // which half-wave (k group of the 32x32 operands)

  // ---- which (head, q-tile) this workgroup owns: head-major, heavy tiles first
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = id / n_qtiles;
  const int qt = CAUSAL ? (n_qtiles - 1 - id % n_qtiles) : (id % n_qtiles);
  const size_t head_off = (size_t)bh * L * D;
  const bf16* qh = q + head_off;
  const bf16* kh = k + head_off;
  const bf16* vh = v + head_off;

  const int q0 = qt * C::BM;               // first row of the workgroup
  const int wrow0 = q0 + wave * 32;         // first row of this wave
  const int my_row = wrow0 + l32;           // the query this lane accumulates

  // ---- Q operand in registers: lane holds d = 16 kc + 8 g + (0..7) of my_row
  bf16x8 qreg[C::KC];
  {
    const bool ok = my_row < L;
    const u32x4* src = reinterpret_cast<const u32x4*>(qh + (size_t)(ok ? my_row : 0) * D + 8 * g);
#pragma unroll
    for (int kc = 0; kc < C::KC; ++kc) {
      u32x4 w = ok ? src[kc * 2] : u32x4{0, 0, 0, 0};
      qreg[kc] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // ---- key tiles this workgroup visits
  const int n_ktiles_all = (L + BN - 1) / BN;
  const int n_kt = CAUSAL ? min(n_ktiles_all, (min(q0 + C::BM, L) - 1) / BN + 1) : n_ktiles_all;

  // global -> register staging of one K and one V tile (rows past L become 0)
  u32x4 kst[C::CPT], vst[C::CPT];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int ci = tid + i * C::THREADS;
      const int r = ci / (D / 8);
      const int cc = ci % (D / 8);
      const int key = kt * BN + r;
      if (key < L) {
        const size_t off = (size_t)key * D + cc * 8;
        kst[i] = *reinterpret_cast<const u32x4*>(kh + off);
        vst[i] = *reinterpret_cast<const u32x4*>(vh + off);
      } else {
        kst[i] = u32x4{0, 0, 0, 0};
        vst[i] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int buf) {
    ATTN_LDS unsigned char* base = smem + buf * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int ci = tid + i * C::THREADS;
      const int r = ci / (D / 8);
      const int cc = ci % (D / 8);
      *reinterpret_cast<ATTN_LDS u32x4*>(base + r * C::PK + cc * 16) = kst[i];
      *reinterpret_cast<ATTN_LDS u32x4*>(base + C::K_BYTES + r * C::PV + cc * 16) = vst[i];
    }
  };

  // ---- running softmax state of my_row (raw-score units) and O^T accumulators
  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};

  const float c = scale * kLog2e;  // exp(scale*(s-m)) == 2^(c*(s-m))

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < n_kt) load_tile(kt + 1);

    const int key0 = kt * BN;
    // a wave whose rows all precede this tile has nothing to do in it
    const bool active = !CAUSAL || key0 <= wrow0 + 31;
    if (active) {
      const ATTN_LDS unsigned char* kb_base = smem + buf * C::STAGE;
      const ATTN_LDS unsigned char* vb_base = kb_base + C::K_BYTES;

      // S^T[key][query] for two 32-key blocks
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
        const ATTN_LDS unsigned char* row = kb_base + (kb * 32 + l32) * C::PK + g * 16;
#pragma unroll
        for (int kc = 0; kc < C::KC; ++kc) {
          bf16x8 a = *reinterpret_cast<const ATTN_LDS bf16x8*>(row + kc * 32);
          s[kb] = mfma32(a, qreg[kc], s[kb]);
        }
      }

      // mask only where the tile reaches past the wave's first row or past L
      const bool need_mask = (CAUSAL && key0 + BN - 1 > wrow0) || (key0 + BN > L);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int key = key0 + kb * 32 + 8 * (j >> 2) + 4 * g + (j & 3);
            const bool vis = (key < L) && (!CAUSAL || key <= my_row);
            s[kb][j] = vis ? s[kb][j] : -INFINITY;
          }
      }

      // row max over this tile: 32 in-lane values, then the other half-wave
      float mt = s[0][0];
#pragma unroll
      for (int j = 1; j < 16; ++j) mt = fmaxf(mt, s[0][j]);
#pragma unroll
      for (int j = 0; j < 16; ++j) mt = fmaxf(mt, s[1][j]);
      mt = max_xor32(mt);
      const float m_new = fmaxf(m_run, mt);

      // rescale l and O only when some row's max grew (wave-uniform branch)
      if (__builtin_amdgcn_ballot_w64(m_new > m_run) != 0) {
        // m_run = -inf gives 0; rows whose max did not move keep alpha = 1
        const float alpha = m_new == m_run ? 1.f : exp2_fast((m_run - m_new) * c);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) acc[db] *= alpha;
        m_run = m_new;
      }
      const float mc = (m_run == -INFINITY ? 0.f : m_run) * c;

      // P = 2^(c s - c m); pack into the bf16 B operands of O^T += V^T P^T
      bf16x8 p[4];
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float e[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            e[i] = exp2_fast(__builtin_fmaf(s[kb][8 * h + i], c, -mc));
            lsum += e[i];
          }
          u32x4 w;
          w[0] = pack_bf16x2(e[0], e[1]);
          w[1] = pack_bf16x2(e[2], e[3]);
          w[2] = pack_bf16x2(e[4], e[5]);
          w[3] = pack_bf16x2(e[6], e[7]);
          p[kb * 2 + h] = __builtin_bit_cast(bf16x8, w);
        }
      l_run += lsum;

      // O^T[d][query] += V^T P^T. Chunk cidx covers keys 16 cidx .. +15; this
      // lane's P elements 0..3 are keys 16 cidx + 4 g + (0..3) and elements 4..7
      // are keys 16 cidx + 8 + 4 g + (0..3) (the S^T accumulator order), so the
      // V^T operand is two transposing reads of 4 keys x 16 columns each.
      const int i16 = lane & 15;
      const int grp = lane >> 4;
#pragma unroll
      for (int cidx = 0; cidx < 4; ++cidx) {
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const int col = db * 32 + (grp & 1) * 16 + 4 * (i16 & 3);
          const int r0 = cidx * 16 + 4 * g + (i16 >> 2);
          const ATTN_LDS bf16x4* a0 =
              reinterpret_cast<const ATTN_LDS bf16x4*>(vb_base + r0 * C::PV + col * 2);
          const ATTN_LDS bf16x4* a1 =
              reinterpret_cast<const ATTN_LDS bf16x4*>(vb_base + (r0 + 8) * C::PV + col * 2);
          bf16x8 a = join(lds_read_tr(a0), lds_read_tr(a1));
          acc[db] = mfma32(a, p[cidx], acc[db]);
        }
      }
    }

    if (kt + 1 < n_kt) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O / l, lse = scale * m + ln l
  const float l_tot = sum_xor32(l_run);
  if (my_row < L) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    bf16* orow = o + head_off + (size_t)my_row * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d = db * 32 + 8 * jj + 4 * g;
        u32x2 w;
        w[0] = pack_bf16x2(acc[db][4 * jj + 0] * inv, acc[db][4 * jj + 1] * inv);
        w[1] = pack_bf16x2(acc[db][4 * jj + 2] * inv, acc[db][4 * jj + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + d) = w;
      }
    if (lse != nullptr && g == 0)
      lse[(size_t)bh * L + my_row] = l_tot > 0.f ? scale * m_run + __logf(l_tot) : -INFINITY;
  }
}

template <int D, int NW, bool CAUSAL>
static hipError_t launch_one(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int H, int L, float scale, hipStream_t stream) {
  using C = PrefillCfg<D, NW>;
  const int n_qtiles = (L + C::BM - 1) / C::BM;
  const long long grid = (long long)B * H * n_qtiles;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const size_t shmem = 2 * C::STAGE;
  auto kern = prefill_bf16_kernel<D, NW, CAUSAL>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::THREADS), shmem, stream,
                     (const bf16*)q, (const bf16*)k, (const bf16*)v, (bf16*)o, lse, B * H, L,
                     n_qtiles, scale);
  return hipGetLastError();
}

hipError_t launch_prefill_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int H, int L, int D, int causal, float scale,
                               hipStream_t stream) {
  if (D == 128) {
    return causal ? launch_one<128, 4, true>(q, k, v, o, lse, B, H, L, scale, stream)
                  : launch_one<128, 4, false>(q, k, v, o, lse, B, H, L, scale, stream);
  }
  return causal ? launch_one<64, 4, true>(q, k, v, o, lse, B, H, L, scale, stream)
                : launch_one<64, 4, false>(q, k, v, o, lse, B, H, L, scale, stream);
}

}  // namespace attn
