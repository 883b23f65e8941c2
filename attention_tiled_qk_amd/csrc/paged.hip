// Paged decode / speculative-verify attention, split-KV merge and paged gather.
//
// What is computed: for each sequence b and head h, the q_len newest queries
// attend all seq_len keys of the sequence (bottom-right causal when asked);
// with grouped-query attention `group` query heads share each KV head h and are
// computed by the same wave from one read of its K/V,
// where token t of the sequence lives in physical block block_tables[b][t/16],
// slot t%16 of the K and V pools -- PagedAttention's block table as [P1] §3.2
// draws it and as the Continuous Batching + PagedAttention item of [P3] passes
// it to the kernel, which reads only the sequence's valid blocks and never the
// slots past seq_len. Long key ranges are cut into splits handled by separate
// workgroups, each producing a normalised partial output and its log-sum-exp,
// and a second kernel merges them (the FlashDecoding item of [P3]).
//
// gfx950 mapping: one wave per (split, head, sequence). Keys are consumed two
// 16-token blocks (32 keys) at a time:
//   * the K slab of a (block, head) is 16 rows x D contiguous; each lane loads
//     its 16-byte pieces straight into the A operand of S^T = K Q^T
//     (v_mfma_f32_16x16x32_bf16; queries, padded to 16, are the N dimension);
//   * the S^T accumulators hold, per lane, one query and 4 keys of each block,
//     so row max / sum are 7 in-lane ops plus two permlane swaps;
//   * P^T goes from those accumulators straight into the B operand of
//     O^T += V^T P^T; V^T comes from the two V slabs written row-major to a
//     per-wave LDS area and read back with ds_read_b64_tr_b16;
//   * block ids are wave-uniform scalar loads; slots past the split's end are
//     masked in S and zeroed in V (a NaN there must not reach O).
//
// FP8 cache (F8): each (block, head) slab holds 16 x D E4M3 codes and one
// float32 scale per pool (the block-wise quantisation of the FlashAttention-3
// item of [P3]; [P2] §五 deploys an FP8 KV cache). A lane loads D/4 contiguous
// code bytes of its K row; the contraction order inside the MFMA is free, so Q
// is loaded in the matching permuted order. Codes become bf16 exactly
// (v_cvt_scalef32_pk_bf16_fp8, scale 1); the K scale multiplies the block's
// scores and the V scale its P, so the cache is read at one byte per value.
#include <type_traits>

#include "common.h"

namespace attn {

constexpr int kIdChunk = 256;  // block ids staged in LDS at a time (even)
constexpr float kMaxPairSum = 1073741824.f;  // 2^30: bound on one lane's P sum per block pair

// WPS waves per workgroup (1, 2 or 4) share one (split, head, sequence): wave
// w takes the w-th part of the split's blocks and the parts are merged in LDS
// at the end, which gives short-split launches more waves without more
// partials.
// Two E4M3 codes (the low or high half of a word) to two bf16, exactly.
__device__ __forceinline__ uint32_t fp8x2_lo(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
}
__device__ __forceinline__ uint32_t fp8x2_hi(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}

// The fp8 variant holds its block pairs as code bytes, half the registers of
// bf16, so it is compiled for three waves per SIMD (measured 2% faster than
// two); the bf16 variant takes what it needs.
template <int D, int WPS, bool F8>
__global__ __launch_bounds__(64 * WPS) __attribute__((amdgpu_waves_per_eu(F8 ? 3 : 1)))
void paged_attn_kernel(
    const bf16* __restrict__ q, const void* __restrict__ k_pool_, const void* __restrict__ v_pool_,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ seq_lens,
    bf16* __restrict__ o, float* __restrict__ lse, float* __restrict__ o_part,
    float* __restrict__ lse_part, int H, int group, int q_len, int max_blocks, int num_splits,
    int causal, float scale, int longest_first) {
  constexpr int DC = D / 32;            // 32-wide chunks of the QK^T contraction
  constexpr int DB = D / 16;            // 16-wide output blocks
  constexpr int PV = D * 2 + 64;        // LDS row pitch of a V slab (bytes)
  constexpr int VCH = 16 * D / 8 / 64;  // 16-byte pieces of one slab per lane
  constexpr int CPR = D / 8;            // 16-byte pieces per slab row
  constexpr int KR = D / 64;            // fp8: 16-byte K pieces per lane (D/4 codes of a row)
  constexpr int VR = D / 64;            // fp8: 16-byte V pieces per lane
  constexpr int CPR8 = D / 16;          // fp8: 16-byte pieces per slab row
  using KV = std::conditional_t<F8, uint8_t, bf16>;
  const KV* k_pool = static_cast<const KV*>(k_pool_);
  const KV* v_pool = static_cast<const KV*>(v_pool_);
  __shared__ __attribute__((aligned(16))) unsigned char vlds_raw[WPS][2 * 16 * PV];
  __shared__ __attribute__((aligned(16))) int ids_raw[WPS][kIdChunk];
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  ATTN_LDS unsigned char* vlds = (ATTN_LDS unsigned char*)vlds_raw[wave];
  ATTN_LDS int* ids = (ATTN_LDS int*)ids_raw[wave];

  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int split = blockIdx.x;
  const int h = blockIdx.y;
  // Longest sequences first (when the host asks for it): workgroups are
  // dispatched in linear-id order (split fastest, sequence slowest), so the z
  // index is taken as a rank and mapped to the sequence of that rank by length
  // (ties by index). The launch then ends on the shortest items instead of on
  // whichever long sequences come last in the batch. One lane holds one
  // length, so this takes batches of up to 64 sequences.
  int b = blockIdx.z;
  if (longest_first && gridDim.z <= 64) {
    const int nseq = gridDim.z;
    const int len = lane < nseq ? seq_lens[lane] : -1;
    int rank = 0;
    for (int j = 0; j < nseq; ++j) {
      const int lj = __builtin_amdgcn_readlane(len, j);
      rank += (lj > len || (lj == len && j < lane)) ? 1 : 0;
    }
    const unsigned long long hit = __builtin_amdgcn_ballot_w64(lane < nseq && rank == (int)blockIdx.z);
    if (hit != 0) b = __builtin_ctzll(hit);
  }

  const int seq_len = seq_lens[b];
  const int nb = (seq_len + 15) >> 4;
  const int per = (nb + num_splits - 1) / num_splits;
  const int blk0 = min(split * per, nb);
  const int blk1 = min(blk0 + per, nb);
  const int key_end = min(seq_len, blk1 * 16);
  const int qpos0 = seq_len - q_len;  // absolute position of query 0
  // Column l16 of the MFMA tiles is query t of query head h * group + gi: the
  // `group` query heads that read KV head h share its K/V loads.
  const int ncols = group * q_len;
  const int t = l16 % q_len;
  const int gi = l16 / q_len;
  const int limit = causal ? qpos0 + t : 0x7fffffff;  // last key my query may see
  // row of (b, query head, query t) in q, o, lse and the partials
  const size_t qrow = (((size_t)b * H + h) * group + (l16 < ncols ? gi : 0)) * q_len + t;

  if (blk0 >= blk1) {  // empty split: contributes nothing to the merge
    if (wave == 0 && l16 < ncols) {
      if (num_splits == 1) {  // only for seq_len == 0, outside the contract
        bf16* dst = o + qrow * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
          *reinterpret_cast<u32x2*>(dst + db * 16 + 4 * g) = u32x2{0u, 0u};
        if (lse != nullptr && g == 0) lse[qrow] = -INFINITY;
      } else {
        float* dst = o_part + (qrow * num_splits + split) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
          *reinterpret_cast<f32x4*>(dst + db * 16 + 4 * g) = f32x4{0.f, 0.f, 0.f, 0.f};
        if (g == 0) lse_part[qrow * num_splits + split] = -INFINITY;
      }
    }
    return;
  }

  // Q as the B operand: lane holds query l16, d = 32 c + 8 g + (0..7). A
  // negative scale is folded into Q (exact sign flip), so the running max is
  // taken over scores that the exponent multiplies by a positive factor.
  const bool neg = scale < 0.f;
  bf16x8 qreg[DC];
  {
    const bool ok = l16 < ncols;
    const unsigned flip = neg ? 0x80008000u : 0u;
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      // contraction slot (c, g, 0..7) holds d = 32c + 8g + i, or for FP8 the
      // lane-contiguous order d = g D/4 + 8c + i that the K loads use
      const int d0 = F8 ? g * (D / 4) + 8 * c : 32 * c + 8 * g;
      u32x4 w = ok ? *reinterpret_cast<const u32x4*>(q + qrow * D + d0) : u32x4{0, 0, 0, 0};
      w ^= flip;
      qreg[c] = __builtin_bit_cast(bf16x8, w);
    }
  }
  const float sc_abs = neg ? -scale : scale;

  const size_t blk_stride = (size_t)H * 16 * D;  // elements per physical block
  const size_t head_off = (size_t)h * 16 * D;
  const int32_t* table = block_tables + (size_t)b * max_blocks;

  float m_run = -INFINITY;
  float mc_run = 0.f;  // cs * m_run, 0 while m_run is unset
  float l_run = 0.f;   // sum of the float32 P: the log-sum-exp
  // bf16 cache: O is divided by the sum of the bf16 P that the PV products use,
  // so the weights applied to V sum to one exactly (dot products of bf16 pairs
  // with (1, 1)). The fp8 kernel folds the V scales into its P and divides by
  // the float32 sum.
  float l_used = 0.f;
  const bf16x2 ones = {(bf16)1.f, (bf16)1.f};
  f32x4 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  // exp(scale*(s-m)) == 2^(cs*(s-m)); cs stays positive so that a masked score
  // (-inf) still gives P = 0 when scale is 0
  const float cs = fmaxf(sc_abs * kLog2e, 1e-30f);

  // K operands (row l16 of each slab) and V pieces (contiguous per instruction)
  // of the block pair n, n+1. A missing second block reads as zeros.
  struct PairB {
    bf16x8 ka[DC], kb[DC];
    u32x4 va[VCH], vb[VCH];
  };
  // FP8: raw code bytes and the two blocks' scales
  struct PairF {
    u32x4 ka[KR], kb[KR], va[VR], vb[VR];
    float ska, skb, sva, svb;
  };
  using Pair = std::conditional_t<F8, PairF, PairB>;
  // the block ids of the current chunk [c0, c1) of this split sit in LDS;
  // an id is read with a wave-uniform LDS load (no wait on global loads)
  int c0 = blk0, c1 = blk0;
  // Both ids of the pair come from one 8-byte LDS read: pairs start at even
  // offsets of the chunk, and when a pair has no second block the chunk has an
  // odd length (kIdChunk is even), so the second entry is still inside ids.
  auto load = [&](int n, Pair& r) {
    const bool has_b = n + 1 < c1;
    const i32x2 pair_ids = *reinterpret_cast<const ATTN_LDS i32x2*>(ids + (n - c0));
    const int pa = __builtin_amdgcn_readfirstlane(pair_ids[0]);
    const int pb_any = __builtin_amdgcn_readfirstlane(pair_ids[1]);
    if constexpr (F8) {
      const uint8_t* ka_src = k_pool + (size_t)pa * blk_stride + head_off;
      const uint8_t* va_src = v_pool + (size_t)pa * blk_stride + head_off;
#pragma unroll
      for (int i = 0; i < KR; ++i)
        r.ka[i] = load_stream(ka_src + l16 * D + g * (D / 4) + 16 * i);
#pragma unroll
      for (int i = 0; i < VR; ++i) r.va[i] = load_stream(va_src + (i * 64 + lane) * 16);
      r.ska = k_scale[(size_t)pa * H + h];
      r.sva = v_scale[(size_t)pa * H + h];
      if (has_b) {
        const int pb = pb_any;
        const uint8_t* kb_src = k_pool + (size_t)pb * blk_stride + head_off;
        const uint8_t* vb_src = v_pool + (size_t)pb * blk_stride + head_off;
#pragma unroll
        for (int i = 0; i < KR; ++i)
          r.kb[i] = load_stream(kb_src + l16 * D + g * (D / 4) + 16 * i);
#pragma unroll
        for (int i = 0; i < VR; ++i) r.vb[i] = load_stream(vb_src + (i * 64 + lane) * 16);
        r.skb = k_scale[(size_t)pb * H + h];
        r.svb = v_scale[(size_t)pb * H + h];
      } else {
#pragma unroll
        for (int i = 0; i < KR; ++i) r.kb[i] = u32x4{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < VR; ++i) r.vb[i] = u32x4{0, 0, 0, 0};
        r.skb = 0.f;
        r.svb = 0.f;
      }
    } else {
    const bf16* ka_src = k_pool + (size_t)pa * blk_stride + head_off;
    const bf16* va_src = v_pool + (size_t)pa * blk_stride + head_off;
#pragma unroll
    for (int c = 0; c < DC; ++c)
      r.ka[c] = __builtin_bit_cast(bf16x8, load_stream(ka_src + l16 * D + 32 * c + 8 * g));
#pragma unroll
    for (int i = 0; i < VCH; ++i) r.va[i] = load_stream(va_src + (i * 64 + lane) * 8);
    if (has_b) {
      const int pb = pb_any;
      const bf16* kb_src = k_pool + (size_t)pb * blk_stride + head_off;
      const bf16* vb_src = v_pool + (size_t)pb * blk_stride + head_off;
#pragma unroll
      for (int c = 0; c < DC; ++c)
        r.kb[c] = __builtin_bit_cast(bf16x8, load_stream(kb_src + l16 * D + 32 * c + 8 * g));
#pragma unroll
      for (int i = 0; i < VCH; ++i) r.vb[i] = load_stream(vb_src + (i * 64 + lane) * 8);
    } else {
#pragma unroll
      for (int c = 0; c < DC; ++c) r.kb[c] = bf16x8{};
#pragma unroll
      for (int i = 0; i < VCH; ++i) r.vb[i] = u32x4{0, 0, 0, 0};
    }
    }
  };

  auto compute = [&](int n, Pair& r) {
    const int key0 = n * 16;
    const bool tail = key0 + 32 > key_end;
    if (tail) {  // V rows at or past the split's end must be exactly zero
      if constexpr (F8) {
#pragma unroll
        for (int i = 0; i < VR; ++i) {
          const int row = (i * 64 + lane) / CPR8;
          if (key0 + row >= key_end) r.va[i] = u32x4{0, 0, 0, 0};
          if (key0 + 16 + row >= key_end) r.vb[i] = u32x4{0, 0, 0, 0};
        }
      } else {
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
          const int row = (i * 64 + lane) / CPR;
          if (key0 + row >= key_end) r.va[i] = u32x4{0, 0, 0, 0};
          if (key0 + 16 + row >= key_end) r.vb[i] = u32x4{0, 0, 0, 0};
        }
      }
    }

    // S^T[key][query] for both blocks
    f32x4 sa = f32x4{0.f, 0.f, 0.f, 0.f}, sb = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (F8) {
      // chunk c is bytes 8c .. 8c+7 of the lane's D/4 codes: two words
      auto kop = [](const u32x4* raw, int c) -> bf16x8 {
        const uint32_t w0 = raw[c >> 1][(c & 1) * 2];
        const uint32_t w1 = raw[c >> 1][(c & 1) * 2 + 1];
        u32x4 o4;
        o4[0] = fp8x2_lo(w0);
        o4[1] = fp8x2_hi(w0);
        o4[2] = fp8x2_lo(w1);
        o4[3] = fp8x2_hi(w1);
        return __builtin_bit_cast(bf16x8, o4);
      };
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        sa = mfma16(kop(r.ka, c), qreg[c], sa);
        sb = mfma16(kop(r.kb, c), qreg[c], sb);
      }
      sa *= r.ska;
      sb *= r.skb;
    } else {
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        sa = mfma16(r.ka[c], qreg[c], sa);
        sb = mfma16(r.kb[c], qreg[c], sb);
      }
    }

    if (tail || (causal && key0 + 31 > qpos0)) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kA = key0 + 4 * g + j;
        const int kB = kA + 16;
        sa[j] = (kA < key_end && kA <= limit) ? sa[j] : -INFINITY;
        sb[j] = (kB < key_end && kB <= limit) ? sb[j] : -INFINITY;
      }
    }

    // P = 2^(cs s - mc) against a reference max m (any m gives the same O and
    // l ratio). The row max is taken, m moved and l, O rescaled only when m is
    // still unset or some lane's P sum over the pair reaches 2^30; otherwise no
    // cross-lane reduction and no rescale run for the pair.
    float e[8];
    auto probs = [&](float mc) -> float {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        e[j] = exp2_fast(__builtin_fmaf(sa[j], cs, -mc));
        e[4 + j] = exp2_fast(__builtin_fmaf(sb[j], cs, -mc));
      }
      return ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
    };
    float ls = probs(mc_run);
    if (__builtin_amdgcn_ballot_w64(!(ls < kMaxPairSum) || m_run == -INFINITY) != 0) {
      float mt = fmaxf(fmaxf(fmaxf(sa[0], sa[1]), fmaxf(sa[2], sa[3])),
                       fmaxf(fmaxf(sb[0], sb[1]), fmaxf(sb[2], sb[3])));
      mt = max_xor16(mt);
      mt = max_xor32(mt);
      const float m_new = fmaxf(m_run, mt);
      // an unchanged m (also -inf == -inf) keeps alpha = 1; m unset before gives 0
      const float alpha = m_new == m_run ? 1.f : exp2_fast((m_run - m_new) * cs);
      l_run *= alpha;
      l_used *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
      m_run = m_new;
      mc_run = (m_run == -INFINITY ? 0.f : m_run) * cs;
      ls = probs(mc_run);
    }
    l_run += ls;
    if constexpr (F8) {  // the V scales of the two blocks go into P
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        e[j] *= r.sva;
        e[4 + j] *= r.svb;
      }
    }
    u32x4 pw;
    pw[0] = pack_bf16x2(e[0], e[1]);
    pw[1] = pack_bf16x2(e[2], e[3]);
    pw[2] = pack_bf16x2(e[4], e[5]);
    pw[3] = pack_bf16x2(e[6], e[7]);
    const bf16x8 p = __builtin_bit_cast(bf16x8, pw);
    if constexpr (!F8) {
      // the pairs as bf16x2 values of the bf16x8 (a pair bit-cast out of a
      // just-written u32x4 element made this compiler keep only the first dot
      // product and scale it by four)
      const bf16x2* pp = reinterpret_cast<const bf16x2*>(&p);
      const float d0 = __builtin_amdgcn_fdot2_f32_bf16(pp[0], ones, 0.f, false);
      const float d1 = __builtin_amdgcn_fdot2_f32_bf16(pp[1], ones, d0, false);
      const float d2 = __builtin_amdgcn_fdot2_f32_bf16(pp[2], ones, 0.f, false);
      const float d3 = __builtin_amdgcn_fdot2_f32_bf16(pp[3], ones, d2, false);
      l_used += d1 + d3;
    }

    // V slabs -> LDS (row-major, padded rows), then transposing reads. The
    // workgroup is this one wave, whose LDS accesses execute in program order,
    // so no barrier is needed (and none may wait for the next pair's loads).
    if constexpr (F8) {  // 16 codes per piece -> 16 bf16 (two 16-byte LDS stores)
      auto widen = [](const u32x4& w, u32x4& lo, u32x4& hi) {
        lo[0] = fp8x2_lo(w[0]);
        lo[1] = fp8x2_hi(w[0]);
        lo[2] = fp8x2_lo(w[1]);
        lo[3] = fp8x2_hi(w[1]);
        hi[0] = fp8x2_lo(w[2]);
        hi[1] = fp8x2_hi(w[2]);
        hi[2] = fp8x2_lo(w[3]);
        hi[3] = fp8x2_hi(w[3]);
      };
#pragma unroll
      for (int i = 0; i < VR; ++i) {
        const int piece = i * 64 + lane;
        const int row = piece / CPR8;
        const int col = piece % CPR8;
        u32x4 lo, hi;
        widen(r.va[i], lo, hi);
        *reinterpret_cast<ATTN_LDS u32x4*>(vlds + row * PV + col * 32) = lo;
        *reinterpret_cast<ATTN_LDS u32x4*>(vlds + row * PV + col * 32 + 16) = hi;
        widen(r.vb[i], lo, hi);
        *reinterpret_cast<ATTN_LDS u32x4*>(vlds + (16 + row) * PV + col * 32) = lo;
        *reinterpret_cast<ATTN_LDS u32x4*>(vlds + (16 + row) * PV + col * 32 + 16) = hi;
      }
    } else {
#pragma unroll
      for (int i = 0; i < VCH; ++i) {
        const int piece = i * 64 + lane;
        const int row = piece / CPR;
        const int col = piece % CPR;
        *reinterpret_cast<ATTN_LDS u32x4*>(vlds + row * PV + col * 16) = r.va[i];
        *reinterpret_cast<ATTN_LDS u32x4*>(vlds + (16 + row) * PV + col * 16) = r.vb[i];
      }
    }
    const ATTN_LDS unsigned char* rd = vlds + (4 * g + (l16 >> 2)) * PV + 8 * (l16 & 3);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const bf16x4 lo = lds_read_tr(reinterpret_cast<const ATTN_LDS bf16x4*>(rd + db * 32));
      const bf16x4 hi = lds_read_tr(reinterpret_cast<const ATTN_LDS bf16x4*>(rd + 16 * PV + db * 32));
      acc[db] = mfma16(join(lo, hi), p, acc[db]);
    }
  };

  // this wave's part of the split: an even number of blocks for every wave
  // but the last, so block pairs never straddle two waves
  const int part = ((blk1 - blk0 + WPS - 1) / WPS + 1) & ~1;
  const int w0 = min(blk0 + wave * part, blk1);
  const int w1 = min(w0 + part, blk1);
  c0 = w0;
  c1 = w0;

  // Chunks of up to kIdChunk blocks (an even number, so block pairs never
  // straddle chunks). Within a chunk the loads are software-pipelined: the
  // K/V of pair n+2 are in flight while pair n is computed.
  for (; c0 < w1; c0 = c1) {
    c1 = min(c0 + kIdChunk, w1);
    for (int i = lane; i < c1 - c0; i += 64) ids[i] = table[c0 + i];
    Pair r0, r1;
    load(c0, r0);
    for (int n = c0;;) {
      if (n + 2 < c1) load(n + 2, r1);
      compute(n, r0);
      n += 2;
      if (n >= c1) break;
      if (n + 2 < c1) load(n + 2, r0);
      compute(n, r1);
      n += 2;
      if (n >= c1) break;
    }
  }

  if constexpr (WPS > 1) {
    // merge the waves' states lane by lane (equal lanes hold the same query,
    // output columns and key positions) into wave 0, through LDS: waves 1 ..
    // WPS-1 leave (m, l, O) in their own staging areas
    static_assert(WPS == 2 || WPS == 4, "two or four waves per split");
    static_assert((3 + 4 * DB) * 64 * sizeof(float) <= sizeof(vlds_raw[0]), "merge staging fits");
    __syncthreads();  // every wave is done with its LDS staging area
    if (wave != 0) {
      float* xw = (float*)vlds_raw[wave];  // (3 + 4 DB) floats per lane
      xw[lane] = m_run;
      xw[64 + lane] = l_run;
      xw[128 + 4 * DB * 64 + lane] = l_used;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) xw[128 + (db * 4 + j) * 64 + lane] = acc[db][j];
    }
    __syncthreads();
    if (wave != 0) return;
    float m_new = m_run;
#pragma unroll
    for (int w = 1; w < WPS; ++w) m_new = fmaxf(m_new, ((const float*)vlds_raw[w])[lane]);
    // an unchanged m (also -inf == -inf) keeps weight 1; an unset m gives 0
    const float a0 = m_run == m_new ? 1.f : exp2_fast((m_run - m_new) * cs);
    l_run *= a0;
    l_used *= a0;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] *= a0;
#pragma unroll
    for (int w = 1; w < WPS; ++w) {
      const float* xw = (const float*)vlds_raw[w];
      const float mw = xw[lane];
      const float aw = mw == m_new ? 1.f : exp2_fast((mw - m_new) * cs);
      l_run += aw * xw[64 + lane];
      l_used += aw * xw[128 + 4 * DB * 64 + lane];
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[db][j] += aw * xw[128 + (db * 4 + j) * 64 + lane];
    }
    m_run = m_new;
  }

  // ---- epilogue
  float l_tot = sum_xor16(l_run);
  l_tot = sum_xor32(l_tot);
  float l_norm = l_tot;
  if constexpr (!F8) {
    l_norm = sum_xor16(l_used);
    l_norm = sum_xor32(l_norm);
  }
  if (l16 < ncols) {
    const float inv = l_norm > 0.f ? 1.f / l_norm : 0.f;
    const float row_lse = l_tot > 0.f ? sc_abs * m_run + __logf(l_tot) : -INFINITY;
    if (num_splits == 1) {
      bf16* dst = o + qrow * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        u32x2 w;
        w[0] = pack_bf16x2(acc[db][0] * inv, acc[db][1] * inv);
        w[1] = pack_bf16x2(acc[db][2] * inv, acc[db][3] * inv);
        *reinterpret_cast<u32x2*>(dst + db * 16 + 4 * g) = w;
      }
      if (lse != nullptr && g == 0) lse[qrow] = row_lse;
    } else {
      float* dst = o_part + (qrow * num_splits + split) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<f32x4*>(dst + db * 16 + 4 * g) = acc[db] * inv;
      if (g == 0) lse_part[qrow * num_splits + split] = row_lse;
    }
  }
}

// Cross-split reduction: one workgroup of D threads per output row. The loops
// over the partials are unrolled by 8 so that their loads are in flight
// together (the kernel is latency-bound: a row is only S (D + 1) floats).
template <int D, typename OutT>
__global__ __launch_bounds__(D) void lse_merge_kernel(const float* __restrict__ o_part,
                                                      const float* __restrict__ lse_part,
                                                      OutT* __restrict__ o, float* __restrict__ lse,
                                                      int S) {
  const size_t row = blockIdx.x;
  const int d = threadIdx.x;
  const float* lp = lse_part + row * S;
  const float* op = o_part + row * S * D + d;
  float m = -INFINITY;
  int p = 0;
  for (; p + 8 <= S; p += 8) {
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = lp[p + i];
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, t[i]);
  }
  for (; p < S; ++p) m = fmaxf(m, lp[p]);
  float acc = 0.f, wsum = 0.f;
  if (m != -INFINITY) {
    for (p = 0; p + 8 <= S; p += 8) {
      float lv[8], ov[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        lv[i] = lp[p + i];
        ov[i] = op[(size_t)(p + i) * D];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float w = lv[i] == -INFINITY ? 0.f : expf(lv[i] - m);
        wsum += w;
        acc = __builtin_fmaf(w, ov[i], acc);
      }
    }
    for (; p < S; ++p) {
      const float lv = lp[p];
      const float w = lv == -INFINITY ? 0.f : expf(lv - m);
      wsum += w;
      acc = __builtin_fmaf(w, op[(size_t)p * D], acc);
    }
  }
  const float out = wsum > 0.f ? acc / wsum : 0.f;
  o[row * D + d] = (OutT)out;
  if (lse != nullptr && d == 0) lse[row] = wsum > 0.f ? m + logf(wsum) : -INFINITY;
}

// Bit-exact copy of each sequence's valid rows out of the pool.
template <int D>
__global__ __launch_bounds__(256) void paged_gather_kernel(const bf16* __restrict__ pool,
                                                           const int32_t* __restrict__ block_tables,
                                                           const int32_t* __restrict__ seq_lens,
                                                           bf16* __restrict__ out, int H,
                                                           int max_blocks, int max_seq_len) {
  constexpr int CPR = D / 8;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int n = min(seq_lens[b], max_seq_len);
  const long long piece = (long long)blockIdx.x * 256 + threadIdx.x;
  const int t = (int)(piece / CPR);
  const int c = (int)(piece % CPR);
  if (t >= n) return;
  const int phys = block_tables[(size_t)b * max_blocks + (t >> 4)];
  const size_t src = (((size_t)phys * H + h) * 16 + (t & 15)) * D + c * 8;
  const size_t dst = (((size_t)b * H + h) * max_seq_len + t) * D + c * 8;
  *reinterpret_cast<u32x4*>(out + dst) = *reinterpret_cast<const u32x4*>(pool + src);
}

struct PagedArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  void* o;
  float* lse;
  float* o_part;
  float* lse_part;
  int H, group, q_len, max_blocks, num_splits, causal;
  float scale;
  int longest_first;
};

template <int D, int WPS, bool F8>
static void launch_paged_variant(dim3 grid, hipStream_t stream, const PagedArgs& a) {
  hipLaunchKernelGGL((paged_attn_kernel<D, WPS, F8>), grid, dim3(64 * WPS), 0, stream,
                     (const bf16*)a.q, a.k_pool, a.v_pool, a.k_scale, a.v_scale, a.block_tables,
                     a.seq_lens, (bf16*)a.o, a.lse, a.o_part, a.lse_part, a.H, a.group, a.q_len,
                     a.max_blocks, a.num_splits, a.causal, a.scale, a.longest_first);
}

template <bool F8>
static void launch_paged_dispatch(int D, int wps, dim3 grid, hipStream_t stream,
                                  const PagedArgs& a) {
  if (D == 128) {
    if (wps == 4) launch_paged_variant<128, 4, F8>(grid, stream, a);
    else if (wps == 2) launch_paged_variant<128, 2, F8>(grid, stream, a);
    else launch_paged_variant<128, 1, F8>(grid, stream, a);
  } else {
    if (wps == 4) launch_paged_variant<64, 4, F8>(grid, stream, a);
    else if (wps == 2) launch_paged_variant<64, 2, F8>(grid, stream, a);
    else launch_paged_variant<64, 1, F8>(grid, stream, a);
  }
}

// k_scale == nullptr: bf16 pools; otherwise E4M3 pools with per-(block, head)
// float32 scales.
hipError_t launch_paged_attn(const void* q, const void* k_pool, const void* v_pool,
                             const float* k_scale, const float* v_scale,
                             const int32_t* block_tables, const int32_t* seq_lens, void* o,
                             float* lse, float* o_part, float* lse_part, int B, int H, int group,
                             int q_len, int D, int max_blocks, int num_splits, int causal,
                             float scale, hipStream_t stream) {
  dim3 grid(num_splits, H, B);
  // With few (split, head, sequence) items the resident waves would leave part
  // of the chip idle in the last round; give each item two waves instead, or
  // four below 1024 items (the grouped-query decode of 64 sequences x 8 KV
  // heads as one split of four waves: 91.7 us, against 97.0 us for two splits
  // of two waves and a merge). The fp8 variant always runs four waves per item
  // (its host side takes an eighth of the automatic splits).
  const long long items = (long long)num_splits * H * B;
  const int wps = k_scale != nullptr ? 4 : items < 1024 ? 4 : items < 4096 ? 2 : 1;
  // Longest-first order pays when splits are long (at least 64 blocks on the
  // widest table): it removes the tail of long items that start late. With
  // short splits it gathers the latency-bound items of short sequences at the
  // end of the launch, where they no longer overlap long streams, and is off.
  const int longest_first = B <= 64 && (max_blocks + num_splits - 1) / num_splits >= 64 ? 1 : 0;
  const PagedArgs a{q, k_pool, v_pool, k_scale, v_scale, block_tables, seq_lens, o, lse, o_part,
                    lse_part, H, group, q_len, max_blocks, num_splits, causal, scale, longest_first};
  if (k_scale != nullptr) launch_paged_dispatch<true>(D, wps, grid, stream, a);
  else launch_paged_dispatch<false>(D, wps, grid, stream, a);
  return hipGetLastError();
}

hipError_t launch_lse_merge(const float* o_part, const float* lse_part, void* o, float* lse,
                            long long rows, int S, int D, int out_bf16, hipStream_t stream) {
  dim3 grid((unsigned)rows);
  if (D == 128) {
    if (out_bf16)
      hipLaunchKernelGGL((lse_merge_kernel<128, bf16>), grid, dim3(128), 0, stream, o_part,
                         lse_part, (bf16*)o, lse, S);
    else
      hipLaunchKernelGGL((lse_merge_kernel<128, float>), grid, dim3(128), 0, stream, o_part,
                         lse_part, (float*)o, lse, S);
  } else {
    if (out_bf16)
      hipLaunchKernelGGL((lse_merge_kernel<64, bf16>), grid, dim3(64), 0, stream, o_part,
                         lse_part, (bf16*)o, lse, S);
    else
      hipLaunchKernelGGL((lse_merge_kernel<64, float>), grid, dim3(64), 0, stream, o_part,
                         lse_part, (float*)o, lse, S);
  }
  return hipGetLastError();
}

hipError_t launch_paged_gather(const void* pool, const int32_t* block_tables,
                               const int32_t* seq_lens, void* out, int B, int H, int D,
                               int max_blocks, int max_seq_len, hipStream_t stream) {
  const long long pieces = (long long)max_seq_len * (D / 8);
  dim3 grid((unsigned)((pieces + 255) / 256), H, B);
  if (D == 128)
    hipLaunchKernelGGL(paged_gather_kernel<128>, grid, dim3(256), 0, stream, (const bf16*)pool,
                       block_tables, seq_lens, (bf16*)out, H, max_blocks, max_seq_len);
  else
    hipLaunchKernelGGL(paged_gather_kernel<64>, grid, dim3(256), 0, stream, (const bf16*)pool,
                       block_tables, seq_lens, (bf16*)out, H, max_blocks, max_seq_len);
  return hipGetLastError();
}

}  // namespace attn
