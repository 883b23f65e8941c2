// Causal / full prefill attention for bf16 Q, K, V on gfx950 matrix cores.
//
// What is computed: O = softmax(scale * Q K^T + mask) V per (batch, head)
// ([P2] §一), by the tiled online-softmax method of [P1] §2.2: Q is cut into
// row tiles (one workgroup each, the query-sequence parallelism that the
// FlashAttention-2 item of [P3] adds), K/V into BN-key tiles streamed through
// LDS; every row keeps a running max m and exp-sum l, and O is divided by l
// once after the last tile. Nothing of size L x L is ever written to memory.
//
// gfx950 mapping (per workgroup of NW waves, BM = 32 * NW query rows):
//   * K/V tiles move HBM -> LDS with buffer_load ... lds (16 bytes per lane, no
//     register round trip). K and V have two LDS stages each: while K_{j+1} and
//     V_j are read, K_{j+2} and V_{j+1} are in flight; one barrier per tile.
//     The buffer range ends at the head's last key (dense: one range per head,
//     tile offsets in the per-lane offset; paged: one per cache-block piece),
//     so rows past L arrive as zeros.
//   * LDS tiles are unpadded; 16-byte chunks are XOR-swizzled per row (a
//     different swizzle for K and for V) so that the K operand reads and the
//     transposing V reads below are free of bank conflicts. The swizzle is
//     applied on the load side by choosing which global chunk each lane fetches.
//   * each wave owns 32 query rows; Q stays in VGPRs as the B operand of
//     S^T = K Q^T (v_mfma_f32_32x32x16_bf16), so every lane's accumulators hold
//     keys of ONE query: row sums are in-lane plus one permlane32 swap, and the
//     O^T accumulator keeps one query per lane too;
//   * P^T feeds O^T += V^T P^T straight from the S^T accumulators (converted to
//     bf16 in registers); V^T operands come from the row-major V tile through
//     ds_read_b64_tr_b16 transposing reads;
//   * software pipelining: iteration j issues the QK^T products of tile j+1 in
//     the same basic block as the exponentials of tile j, so one wave's matrix
//     cores and vector ALUs work at the same time;
//   * reference max: any reference m gives the same O = sum(e^(s-m) v) /
//     sum(e^(s-m)). m is set from each row's first tile before the loop; the
//     exponentials use the current m, and only when a lane's P sum over a tile
//     reaches 2^30 is the row max taken, m moved, l and O rescaled and P
//     recomputed -- rare;
//   * causal: key tiles above a wave's last row are skipped, the mask is only
//     evaluated on tiles that cross the diagonal, and the work order (tile_of)
//     keeps each head on one XCD and starts the longest query tiles first;
//     launches with evenly loaded tiles (full attention, paged chunks) run a
//     head's query tiles side by side instead (tile_of_head_major);
//   * epilogue: O leaves through LDS (the idle K stages) as whole 128-byte
//     lines with streaming stores, so it drains during the launch.
#include <type_traits>

#include "common.h"

namespace attn {

namespace {

constexpr float kMaxTileSum = 1073741824.f;   // 2^30: bound on one lane's P sum per tile
constexpr int kPagedMaxBlocks = 2048;         // cache blocks per sequence (32768 keys) in paged mode

template <int D, int NW, int BN>
struct PrefillCfg {
  static constexpr int BM = 32 * NW;        // query rows per workgroup
  static constexpr int KC = D / 16;         // 16-wide k chunks of the QK^T contraction
  static constexpr int DB = D / 32;         // 32-wide output column blocks
  static constexpr int NCH = D / 8;         // 16-byte chunks per K/V row
  static constexpr int ROWB = 2 * D;        // bytes per K/V row
  static constexpr int TILEB = BN * ROWB;   // bytes per K (or V) tile
  static constexpr int PIECES = TILEB / 1024;
  static constexpr int PPW = PIECES / NW;   // 1 KB pieces per wave per tile (K or V)
  static constexpr int RPP = 1024 / ROWB;   // rows per piece
  static constexpr int NKB = BN / 32;       // 32-key blocks per tile
  static constexpr int LOADS = 2 * PPW;     // buffer loads per wave per tile
  static constexpr int THREADS = NW * 64;
  static_assert(PIECES % NW == 0 && PPW >= 1, "tile pieces must split evenly over the waves");
  static_assert(BN % 32 == 0, "key tile is a multiple of 32");
};

// Swizzle of the 16-byte chunk index within a K row: chunk c of row r is stored
// at c ^ kswz(r). Sixteen consecutive rows (one 16-lane group of the K operand
// read) then cover all 64 banks: at D = 128 a row is one bank sweep and the
// chunk moves with r; at D = 64 two rows share a sweep and it moves with r / 2.
template <int NCH>
__device__ __forceinline__ int kswz(int r) { return (NCH == 16 ? r : r >> 1) & (NCH - 1); }
// V rows: the transposing read touches 8 consecutive rows x 4 chunks; rows
// r & 3 go to different 64-byte groups and (r >> 2) & 1 permutes within them.
template <int NCH>
__device__ __forceinline__ int vswz(int r) { return (((r & 3) << 2) | ((r >> 2) & 1)) & (NCH - 1); }

// Work item of workgroup `id`: (head bh, query tile qt). The dispatcher hands
// workgroup ids to the 8 XCDs in turn (id % 8), each XCD starting them in id
// order. When the head count splits evenly, XCD x owns a contiguous group of
// heads (their K/V share its L2) and starts the longest causal tiles of all
// its heads first, the shortest last, so the tail of the launch is short work.
__device__ __forceinline__ void tile_of(int id, int n_heads, int n_qtiles, int& bh, int& qt) {
  if ((n_heads & 7) == 0) {
    const int hpx = n_heads >> 3;
    const int pos = id >> 3;
    qt = n_qtiles - 1 - pos / hpx;
    bh = (id & 7) * hpx + pos % hpx;
  } else {
    qt = n_qtiles - 1 - id / n_heads;
    bh = id % n_heads;
  }
}

// Head-major work order, for launches whose query tiles carry similar work
// (full attention; a chunk after a long cached prefix): the query tiles of one
// head get consecutive ids on the same XCD, so they run together and stream
// that head's K/V through its L2 once instead of once per tile.
__device__ __forceinline__ void tile_of_head_major(int id, int n_heads, int n_qtiles, int& bh,
                                                   int& qt) {
  if ((n_heads & 7) == 0) {
    const int hpx = n_heads >> 3;
    const int pos = id >> 3;
    bh = (id & 7) * hpx + pos / n_qtiles;
    qt = n_qtiles - 1 - pos % n_qtiles;
  } else {
    bh = id / n_qtiles;
    qt = n_qtiles - 1 - id % n_qtiles;
  }
}

}  // namespace

// Where the keys come from when the kernel runs over a paged cache: the
// queries are the q_len newest tokens of each sequence (chunked prefill), the
// keys are its seq_lens[b] cached tokens read through its block table. With
// cu_q set, sequences have their own query counts (a ragged batch): sequence b
// owns packed query tokens cu_q[b] .. cu_q[b+1]-1, and q, o and lse are laid
// out token-major ([total_q, heads, D] and [total_q, heads]).
struct PagedKV {
  const int32_t* block_tables;  // [B, max_blocks]
  const int32_t* seq_lens;      // [B], keys per sequence including its new tokens
  const int32_t* cu_q;          // [B + 1] packed query offsets, or null (q_len = L for all)
  int heads;                    // query heads per sequence
  int max_blocks;
  int kv_heads;                 // heads of the pools; query head h reads h / (heads / kv_heads)
  int pool_bytes;               // bytes of each pool when below 2^31 (one buffer range each), else 0
};

template <int D, int NW, int BN, bool CAUSAL, bool PAGED = false, bool POOL = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void prefill_bf16_pipe_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    bf16* __restrict__ o, float* __restrict__ lse, int L, int n_heads, int n_qtiles, float scale,
    PagedKV pg) {
  using C = PrefillCfg<D, NW, BN>;
  __shared__ __attribute__((aligned(1024))) unsigned char ks0[C::TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char ks1[C::TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char vs0[C::TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char vs1[C::TILEB];
  __shared__ __attribute__((aligned(16))) int ids[PAGED ? kPagedMaxBlocks : 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int g = lane >> 5;

  int bh, qt;
  if (CAUSAL && !PAGED) tile_of(blockIdx.x, n_heads, n_qtiles, bh, qt);
  else tile_of_head_major(blockIdx.x, n_heads, n_qtiles, bh, qt);
  // L queries per head; Lk keys, the last L of which are the queries' own
  // positions (Lk == L for dense prefill). Query row r sits at position off + r.
  const size_t head_off = (size_t)bh * L * D;  // dense K, V of this head
  const bf16* kh = k + head_off;
  const bf16* vh = v + head_off;
  size_t qo_off = head_off;       // Q, O row 0 of this head
  size_t row_stride = D;          // elements between consecutive query rows
  size_t lse_off = (size_t)bh * L;
  size_t lse_stride = 1;
  int Lk = L, hh = 0, kvh = 0, seq = 0;
  if constexpr (PAGED) {
    seq = bh / pg.heads;
    hh = bh - seq * pg.heads;
    kvh = hh / (pg.heads / pg.kv_heads);
    Lk = pg.seq_lens[seq];
    if (pg.cu_q != nullptr) {
      const int c0 = pg.cu_q[seq];
      L = pg.cu_q[seq + 1] - c0;
      if (qt * C::BM >= L) return;  // whole workgroup: past this sequence's queries
      qo_off = ((size_t)c0 * pg.heads + hh) * D;
      row_stride = (size_t)pg.heads * D;
      lse_off = (size_t)c0 * pg.heads + hh;
      lse_stride = pg.heads;
    }
  }
  const int off = Lk - L;

  const int q0 = qt * C::BM;
  const int wrow0 = q0 + wave * 32;
  const int my_row = wrow0 + l32;
  const int n_kt = CAUSAL ? (off + min(q0 + C::BM, L) - 1) / BN + 1 : (Lk + BN - 1) / BN;
  // last key tile holding a key that some row of this wave may see
  const int last_w = CAUSAL ? min(n_kt - 1, (off + wrow0 + 31) / BN) : n_kt - 1;

  // Per-lane source offsets of the tile loads: relative to the tile (dense) or
  // to the piece's first row (paged: a piece's RPP rows are consecutive slots of
  // one cache block, contiguous in the pool). Piece i of this wave starts
  // NW * RPP rows (4096 bytes) after piece i - 1 and both swizzles repeat every
  // 16 rows, so one offset per lane serves every piece: the piece's own position
  // is added to it (dense, and paged pools below 2 GiB) or is the start of the
  // piece's buffer range (larger pools).
  static_assert(NW * C::RPP * C::ROWB == 4096, "piece stride");
  unsigned koff, voff;
  {
    const int row = wave * C::RPP + lane / C::NCH;
    const int phys = lane % C::NCH;
    const int base = PAGED ? (lane / C::NCH) * C::ROWB : row * C::ROWB;
    koff = base + (phys ^ kswz<C::NCH>(row)) * 16;
    voff = base + (phys ^ vswz<C::NCH>(row)) * 16;
  }
  if constexpr (PAGED) {
    // stage this sequence's block ids once; reading them back from LDS keeps
    // global loads (which complete in order) out of the prefetch pipeline
    const int nb = min((Lk + 15) >> 4, pg.max_blocks);
    const int32_t* tab = pg.block_tables + (size_t)seq * pg.max_blocks;
    for (int i = tid; i < nb; i += NW * 64) ids[i] = tab[i];
    __syncthreads();
  }
  auto kst = [&](auto s) -> ATTN_LDS unsigned char* {
    if constexpr (decltype(s)::value == 0) return (ATTN_LDS unsigned char*)ks0;
    else return (ATTN_LDS unsigned char*)ks1;
  };
  auto vst = [&](auto s) -> ATTN_LDS unsigned char* {
    if constexpr (decltype(s)::value == 0) return (ATTN_LDS unsigned char*)vs0;
    else return (ATTN_LDS unsigned char*)vs1;
  };
  // paged: a key tile (BN = 64 keys) spans exactly four cache blocks, ids
  // 4 kt .. 4 kt + 3, read with one 16-byte LDS load (index at most 2047, since
  // Lk <= 16 kPagedMaxBlocks; entries past the sequence's blocks are never
  // used). One load and one wait per tile instead of one per 1 KiB piece.
  static_assert(!PAGED || BN == 64, "a paged key tile spans four cache blocks");
  auto tile_blocks = [&](int kt) -> i32x4 { return *reinterpret_cast<const i32x4*>(ids + 4 * kt); };
  // the buffer range of piece i of tile kt -- the piece's rows inside their
  // cache block, ending at the sequence's last key (rows past it, and pieces
  // wholly past it, read as zeros). The block is chosen among the tile's four
  // by value selects (no indexed access, which would go through scratch).
  auto paged_piece = [&](const bf16* pool, int kt, int i, i32x4 bl) -> __amdgpu_buffer_rsrc_t {
    const int off_in_tile = (wave + NW * i) * C::RPP;
    const int key = kt * BN + off_in_tile;
    const int which = off_in_tile >> 4;  // 0 .. 3, wave-uniform
    const int lo = (which & 1) ? bl[1] : bl[0];
    const int hi = (which & 1) ? bl[3] : bl[2];
    const int id = __builtin_amdgcn_readfirstlane((which & 2) ? hi : lo);
    const bool live = key < Lk;
    const bf16* src = pool + (((size_t)(live ? id : 0) * pg.kv_heads + kvh) * 16 + (key & 15)) * D;
    return buffer_rsrc(src, live ? min(C::RPP, Lk - key) * C::ROWB : 0);
  };
  // Dense source: one buffer range per head, its L rows of K or V. The tile and
  // piece offsets ride in the per-lane offset (soffset stays 0), which the
  // range check covers, so rows past L read as zeros; per piece the issue is one
  // vector add instead of a descriptor built on the scalar unit.
  const __amdgpu_buffer_rsrc_t k_head = buffer_rsrc(kh, PAGED ? 0 : L * C::ROWB);
  const __amdgpu_buffer_rsrc_t v_head = buffer_rsrc(vh, PAGED ? 0 : L * C::ROWB);
  // Paged, pools below 2 GiB: one buffer range per pool. A piece's cache-block
  // offset (a few scalar instructions) and the lane's row in the piece ride in
  // the per-lane offset; lanes whose key is past the sequence's end take an
  // offset beyond the range and read zeros.
  const __amdgpu_buffer_rsrc_t k_pool_rs = buffer_rsrc(k, POOL ? pg.pool_bytes : 0);
  const __amdgpu_buffer_rsrc_t v_pool_rs = buffer_rsrc(v, POOL ? pg.pool_bytes : 0);
  const int lane_row = lane / C::NCH;
  // `full`: the whole tile lies before the sequence's end (wave-uniform), so
  // no lane needs the range check (all but the last tile of a sequence)
  auto pool_off = [&](int kt, int i, i32x4 bl, unsigned lane_off, bool full) -> unsigned {
    const int off_in_tile = (wave + NW * i) * C::RPP;
    const int key = kt * BN + off_in_tile;
    const int which = off_in_tile >> 4;  // 0 .. 3, wave-uniform
    const int lo = (which & 1) ? bl[1] : bl[0];
    const int hi = (which & 1) ? bl[3] : bl[2];
    const unsigned id = (unsigned)__builtin_amdgcn_readfirstlane((which & 2) ? hi : lo);
    const unsigned base = ((id * (unsigned)pg.kv_heads + (unsigned)kvh) * 16u + (unsigned)(key & 15)) * (unsigned)C::ROWB;
    if (full) return base + lane_off;
    return lane_row < Lk - key ? base + lane_off : 0x80000000u;
  };
  auto issue_k = [&](auto s, int kt) {
    if constexpr (PAGED && POOL) {
      const i32x4 bl = tile_blocks(kt);
      if (kt * BN + BN <= Lk) {
#pragma unroll
        for (int i = 0; i < C::PPW; ++i) dma16(k_pool_rs, kst(s) + (wave + NW * i) * 1024, pool_off(kt, i, bl, koff, true));
      } else {
#pragma unroll
        for (int i = 0; i < C::PPW; ++i) dma16(k_pool_rs, kst(s) + (wave + NW * i) * 1024, pool_off(kt, i, bl, koff, false));
      }
    } else if constexpr (PAGED) {
      const i32x4 bl = tile_blocks(kt);
#pragma unroll
      for (int i = 0; i < C::PPW; ++i) dma16(paged_piece(k, kt, i, bl), kst(s) + (wave + NW * i) * 1024, koff);
    } else {
#pragma unroll
      for (int i = 0; i < C::PPW; ++i)
        dma16(k_head, kst(s) + (wave + NW * i) * 1024, koff + (unsigned)((kt * BN + NW * C::RPP * i) * C::ROWB));
    }
  };
  auto issue_v = [&](auto s, int kt) {
    if constexpr (PAGED && POOL) {
      const i32x4 bl = tile_blocks(kt);
      if (kt * BN + BN <= Lk) {
#pragma unroll
        for (int i = 0; i < C::PPW; ++i) dma16(v_pool_rs, vst(s) + (wave + NW * i) * 1024, pool_off(kt, i, bl, voff, true));
      } else {
#pragma unroll
        for (int i = 0; i < C::PPW; ++i) dma16(v_pool_rs, vst(s) + (wave + NW * i) * 1024, pool_off(kt, i, bl, voff, false));
      }
    } else if constexpr (PAGED) {
      const i32x4 bl = tile_blocks(kt);
#pragma unroll
      for (int i = 0; i < C::PPW; ++i) dma16(paged_piece(v, kt, i, bl), vst(s) + (wave + NW * i) * 1024, voff);
    } else {
#pragma unroll
      for (int i = 0; i < C::PPW; ++i)
        dma16(v_head, vst(s) + (wave + NW * i) * 1024, voff + (unsigned)((kt * BN + NW * C::RPP * i) * C::ROWB));
    }
  };

  // LDS operand addresses. Chunk 2 kc + g of K row l32 sits at chunk
  // (2 kc + g) ^ kswz(l32) = (2 kc) ^ (g ^ kswz(l32)), so the address of k-chunk
  // kc is that of chunk 0 XOR 32 kc; likewise V column block db is block 0
  // XOR 64 db. One register each instead of one per chunk.
  const int kaddr0 = l32 * C::ROWB + ((g ^ kswz<C::NCH>(l32)) * 16);
  int vaddr0;
  {
    const int i16 = lane & 15;
    const int grp = lane >> 4;
    const int r = 4 * g + (i16 >> 2);
    const int c = 2 * (grp & 1) + ((i16 & 3) >> 1);
    vaddr0 = r * C::ROWB + ((c ^ vswz<C::NCH>(r)) * 16) + 8 * (i16 & 1);
  }

  const bool neg = scale < 0.f;
  const float sc_abs = neg ? -scale : scale;
  bf16x8 qreg[C::KC];
  // Q: all loads issued together from a valid row (a row past L reads row 0
  // and is zeroed after the load, by a select rather than a branch around the
  // load: the branches let the compiler wait on the first loads before issuing
  // the rest and the K/V tiles), then the first K/V tiles, then the sign flip
  // and the zeroing, which wait for the Q data.
  const bool q_ok = my_row < L;
  u32x4 qraw[C::KC];
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(q + qo_off + (q_ok ? my_row : 0) * row_stride + 8 * g);
#pragma unroll
    for (int kc = 0; kc < C::KC; ++kc) qraw[kc] = src[kc * 2];
  }

  issue_k(std::integral_constant<int, 0>{}, 0);
  issue_v(std::integral_constant<int, 0>{}, 0);
  if (n_kt > 1) issue_k(std::integral_constant<int, 1>{}, 1);
  {
    const unsigned flip = neg ? 0x80008000u : 0u;
    const unsigned keep = q_ok ? 0xffffffffu : 0u;
#pragma unroll
    for (int kc = 0; kc < C::KC; ++kc) qreg[kc] = __builtin_bit_cast(bf16x8, (qraw[kc] & keep) ^ flip);
  }

  float m_run = -INFINITY;  // reference max (raw-score units)
  float mc_run = 0.f;       // c * m_run, 0 while m_run is unset
  float l_run = 0.f;
  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};
  // exp(scale*(s-m)) == 2^(c*(s-m)); c is kept positive so that a masked score
  // (-inf) still gives P = 0 when scale is 0 (c*s then underflows to 0)
  const float c = fmaxf(sc_abs * kLog2e, 1e-30f);

  auto qk = [&](f32x16* sc, const ATTN_LDS unsigned char* kb_) {
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) {
      sc[kb] = f32x16{};
#pragma unroll
      for (int kc = 0; kc < C::KC; ++kc) {
        const bf16x8 a = *reinterpret_cast<const ATTN_LDS bf16x8*>(kb_ + (kaddr0 ^ (32 * kc)) + kb * 32 * C::ROWB);
        sc[kb] = mfma32(a, qreg[kc], sc[kb]);
      }
    }
  };
  auto mask = [&](f32x16* sc, int kt) {
    const int key0 = kt * BN;
    const bool need_mask = CAUSAL ? (key0 + BN - 1 > off + wrow0) : (key0 + BN > Lk);
    if (need_mask) {
      const int lim = (CAUSAL ? off + my_row : Lk - 1) - key0 - 4 * g;
      // last key that the wave's first / last row sees (wave-uniform): a
      // 32-key block wholly below the first is left alone, one wholly above the
      // last is cleared, only a block in between is masked key by key
      const int lo = CAUSAL ? off + wrow0 : Lk - 1;
      const int hi = CAUSAL ? off + wrow0 + 31 : Lk - 1;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
        const int kfirst = key0 + 32 * kb;
        if (kfirst + 31 <= lo) continue;
        if (kfirst > hi) {
#pragma unroll
          for (int j = 0; j < 16; ++j) sc[kb][j] = -INFINITY;
          continue;
        }
#pragma unroll
        for (int j = 0; j < 16; ++j)
          sc[kb][j] = (kb * 32 + 8 * (j >> 2) + (j & 3) <= lim) ? sc[kb][j] : -INFINITY;
      }
    }
  };
  // P = 2^(c s - mc) as the bf16 B operands of O^T += V^T P^T; returns this
  // lane's sum of P over the tile
  auto probs = [&](const f32x16* sc, bf16x8* p, float mc) -> float {
    float part[2 * C::NKB];
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = exp2_fast(__builtin_fmaf(sc[kb][8 * h + i], c, -mc));
        part[2 * kb + h] = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
        u32x4 w;
        w[0] = pack_bf16x2(e[0], e[1]);
        w[1] = pack_bf16x2(e[2], e[3]);
        w[2] = pack_bf16x2(e[4], e[5]);
        w[3] = pack_bf16x2(e[6], e[7]);
        p[2 * kb + h] = __builtin_bit_cast(bf16x8, w);
      }
    float lsum = part[0];
#pragma unroll
    for (int i = 1; i < 2 * C::NKB; ++i) lsum += part[i];
    return lsum;
  };
  // Moves the reference max m to the running row maximum including this tile
  // and returns the factor that l and O must be scaled by.
  auto move_max = [&](const f32x16* sc) -> float {
    float mt = sc[0][0];
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
      for (int j = (kb == 0 ? 1 : 0); j < 16; ++j) mt = fmaxf(mt, sc[kb][j]);
    mt = max_xor32(mt);
    const float m_new = fmaxf(m_run, mt);
    // an unchanged m (also -inf == -inf) gives 1; m = -inf before gives 0
    const float alpha = m_new == m_run ? 1.f : exp2_fast((m_run - m_new) * c);
    m_run = m_new;
    mc_run = (m_run == -INFINITY ? 0.f : m_run) * c;
    return alpha;
  };
  // Softmax of one tile into P. The exponents use the current reference m; only
  // when some lane's P sum reaches 2^30 (scores grew by 30 / c past m, or m is
  // still unset) is the row maximum taken, m moved and P recomputed. Any m gives
  // the same O and l ratio, and P below 2^30 keeps l, O and the bf16 P finite.
  auto softmax = [&](const f32x16* sc, bf16x8* p) {
    float ls = probs(sc, p, mc_run);
    if (__builtin_amdgcn_ballot_w64(!(ls < kMaxTileSum) || m_run == -INFINITY) != 0) {
      const float alpha = move_max(sc);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) acc[db] *= alpha;
      ls = probs(sc, p, mc_run);
    }
    l_run += ls;
  };
  auto pv = [&](const bf16x8* p, const ATTN_LDS unsigned char* vb_) {
#pragma unroll
    for (int cidx = 0; cidx < 2 * C::NKB; ++cidx) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const ATTN_LDS unsigned char* base = vb_ + (vaddr0 ^ (64 * db)) + cidx * 16 * C::ROWB;
        const bf16x4 lo = lds_read_tr(reinterpret_cast<const ATTN_LDS bf16x4*>(base));
        const bf16x4 hi = lds_read_tr(reinterpret_cast<const ATTN_LDS bf16x4*>(base + 8 * C::ROWB));
        acc[db] = mfma32(join(lo, hi), p[cidx], acc[db]);
      }
    }
    // Issue order of this block: 12 transposing V reads ahead, then one product
    // per two reads (left to itself the scheduler keeps about 4 in flight and
    // each product waits on its read; A/B: c2 -2.4%, cpf -4.4%, c3 -0.4%)
    constexpr int AHEAD = 12;
    constexpr int NMF = 2 * C::NKB * C::DB;
    static_assert(AHEAD % 2 == 0 && AHEAD <= 2 * NMF, "reads ahead");
    __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);  // DS reads
#pragma unroll
    for (int i = 0; i < NMF; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      if (2 * (i + 1) + AHEAD <= 2 * NMF) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };

  f32x16 sa[C::NKB], sb[C::NKB];
  wait_vmcnt<0>();
  lds_barrier();
  qk(sa, kst(std::integral_constant<int, 0>{}));
  // the reference of every row is set from its first tile here, before the
  // pipelined loop, so that tile takes the common path (one pass of
  // exponentials, no rescale of the still-zero l and O)
  mask(sa, 0);
  (void)move_max(sa);

  // Iteration j (every wave takes part in its barrier and loads): tile j's
  // scores are in s_cur, K_{j+1} and V_j are in LDS. The loop is split by
  // wave-uniform phase -- tiles before the wave's last visible tile, that tile,
  // and tiles past it -- so that the hot body has no branch between the
  // products of tile j+1 and the softmax of tile j.
  auto sync_and_load = [&](auto par, int j) {
    constexpr int P = decltype(par)::value;
    wait_vmcnt<0>();
    lds_barrier();
    if (j + 2 < n_kt) issue_k(std::integral_constant<int, P>{}, j + 2);
    if (j + 1 < n_kt) issue_v(std::integral_constant<int, 1 - P>{}, j + 1);
  };
  auto full = [&](auto par, int j, f32x16* s_cur, f32x16* s_nxt) {
    constexpr int P = decltype(par)::value;
    sync_and_load(par, j);
    mask(s_cur, j);
    // products of tile j+1 and the softmax of tile j share one basic block
    bf16x8 p[2 * C::NKB];
    qk(s_nxt, kst(std::integral_constant<int, 1 - P>{}));
    softmax(s_cur, p);
    pv(p, vst(std::integral_constant<int, P>{}));
  };
  auto last = [&](auto par, int j, f32x16* s_cur) {
    constexpr int P = decltype(par)::value;
    sync_and_load(par, j);
    mask(s_cur, j);
    bf16x8 p[2 * C::NKB];
    softmax(s_cur, p);
    pv(p, vst(std::integral_constant<int, P>{}));
  };

  int j = 0;
  for (; j + 1 < last_w; j += 2) {
    full(std::integral_constant<int, 0>{}, j, sa, sb);
    full(std::integral_constant<int, 1>{}, j + 1, sb, sa);
  }
  if (j < last_w) {
    full(std::integral_constant<int, 0>{}, j, sa, sb);
    last(std::integral_constant<int, 1>{}, j + 1, sb);
    j += 2;
  } else {
    last(std::integral_constant<int, 0>{}, j, sa);
    j += 1;
  }
  for (; j < n_kt; ++j) {
    if (j & 1) sync_and_load(std::integral_constant<int, 1>{}, j);
    else sync_and_load(std::integral_constant<int, 0>{}, j);
  }

  const float l_tot = sum_xor32(l_run);
  // O goes through the K stages, idle once every wave has passed the barrier
  // below: written in the accumulator layout with each row's 16-byte chunks
  // XOR-swizzled (conflict-free both ways), read back row-major, and stored 16
  // bytes per lane so that 8 lanes write a whole 128-byte line, with the
  // streaming (nontemporal) policy: the lines leave the L2 during the launch
  // instead of in the write-back at its end.
  lds_barrier();
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int wbyte = wave * 32 * C::ROWB;
  ATTN_LDS unsigned char* ob = wbyte < C::TILEB ? kst(std::integral_constant<int, 0>{}) + wbyte
                                                : kst(std::integral_constant<int, 1>{}) + (wbyte - C::TILEB);
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int c = db * 4 + jj;
      u32x2 w;
      w[0] = pack_bf16x2(acc[db][4 * jj + 0] * inv, acc[db][4 * jj + 1] * inv);
      w[1] = pack_bf16x2(acc[db][4 * jj + 2] * inv, acc[db][4 * jj + 3] * inv);
      *reinterpret_cast<ATTN_LDS u32x2*>(ob + l32 * C::ROWB + ((c ^ (l32 & (C::NCH - 1))) * 16) + 8 * g) = w;
    }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
  constexpr int RPI = 64 / C::NCH;      // rows per store instruction
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = RPI * i + lane / C::NCH;
    const int c = lane % C::NCH;
    const u32x4 w = *reinterpret_cast<const ATTN_LDS u32x4*>(ob + r * C::ROWB + ((c ^ (r & (C::NCH - 1))) * 16));
    const int grow = wrow0 + r;
    if (grow < L) __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(o + qo_off + grow * row_stride + c * 8));
  }
  if (my_row < L && lse != nullptr && g == 0)
    lse[lse_off + my_row * lse_stride] = l_tot > 0.f ? sc_abs * m_run + __logf(l_tot) : -INFINITY;
}

template <int D, int NW, int BN, bool CAUSAL, bool PAGED = false, bool POOL = false>
hipError_t launch_prefill_pipe(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int H, int L, float scale, hipStream_t stream,
                               PagedKV pg = PagedKV{nullptr, nullptr, nullptr, 0, 0, 0, 0}) {
  using C = PrefillCfg<D, NW, BN>;
  const int n_qtiles = (L + C::BM - 1) / C::BM;
  const long long grid = (long long)B * H * n_qtiles;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_bf16_pipe_kernel<D, NW, BN, CAUSAL, PAGED, POOL>), dim3((unsigned)grid),
                     dim3(C::THREADS), 0, stream, (const bf16*)q, (const bf16*)k, (const bf16*)v,
                     (bf16*)o, lse, L, B * H, n_qtiles, scale, pg);
  return hipGetLastError();
}

// Query rows per workgroup of the configuration launch_prefill_bf16 uses.
int prefill_bf16_rows() { return 128; }

// Longest sequence (in cache blocks) launch_paged_prefill_bf16 accepts.
int paged_prefill_max_blocks() { return kPagedMaxBlocks; }

hipError_t launch_prefill_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int H, int L, int D, int causal, float scale,
                               hipStream_t stream) {
  if (D == 128) {
    return causal ? launch_prefill_pipe<128, 4, 64, true>(q, k, v, o, lse, B, H, L, scale, stream)
                  : launch_prefill_pipe<128, 4, 64, false>(q, k, v, o, lse, B, H, L, scale, stream);
  }
  return causal ? launch_prefill_pipe<64, 4, 64, true>(q, k, v, o, lse, B, H, L, scale, stream)
                : launch_prefill_pipe<64, 4, 64, false>(q, k, v, o, lse, B, H, L, scale, stream);
}

hipError_t launch_paged_prefill_bf16(const void* q, const void* k_pool, const void* v_pool,
                                     const int32_t* block_tables, const int32_t* seq_lens, void* o,
                                     float* lse, int B, int H, int q_len, int D, int max_blocks,
                                     int causal, float scale, hipStream_t stream,
                                     const int32_t* cu_q, int Hkv, int num_blocks) {
  // with cu_q, q_len is the longest sequence's query count (it sizes the grid);
  // H query heads read the pools' Hkv heads in groups of H / Hkv
  const long long pool_bytes = (long long)num_blocks * Hkv * 16 * D * 2;
  const bool pool32 = pool_bytes < 0x80000000LL;
  const PagedKV pg{block_tables, seq_lens, cu_q, H, max_blocks, Hkv, pool32 ? (int)pool_bytes : 0};
  auto go = [&](auto d, auto c, auto p) {
    constexpr int DD = decltype(d)::value;
    constexpr bool CC = decltype(c)::value;
    constexpr bool PP = decltype(p)::value;
    return launch_prefill_pipe<DD, 4, 64, CC, true, PP>(q, k_pool, v_pool, o, lse, B, H, q_len, scale,
                                                        stream, pg);
  };
  using D128 = std::integral_constant<int, 128>;
  using D64 = std::integral_constant<int, 64>;
  using T = std::true_type;
  using F = std::false_type;
  if (D == 128) {
    if (causal) return pool32 ? go(D128{}, T{}, T{}) : go(D128{}, T{}, F{});
    return pool32 ? go(D128{}, F{}, T{}) : go(D128{}, F{}, F{});
  }
  if (causal) return pool32 ? go(D64{}, T{}, T{}) : go(D64{}, T{}, F{});
  return pool32 ? go(D64{}, F{}, T{}) : go(D64{}, F{}, F{});
}

}  // namespace attn
