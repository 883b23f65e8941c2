// Device-side helpers shared by the gfx950 attention kernels.
//
// Matrix-core layouts used throughout (gfx950, wave64; checked on the device):
//   v_mfma_f32_32x32x16_bf16  C[32x32] += A[32x16] B[16x32]
//     A: lane l holds row l%32, k = 8*(l/32) + e   (e = 0..7, one 16-byte operand)
//     B: lane l holds col l%32, k = 8*(l/32) + e
//     C: lane l holds col l%32, rows 8*(j/4) + 4*(l/32) + j%4   (j = 0..15)
//   v_mfma_f32_16x16x32_bf16  C[16x16] += A[16x32] B[32x16]
//     A: lane l holds row l%16, k = 8*(l/16) + e
//     B: lane l holds col l%16, k = 8*(l/16) + e
//     C: lane l holds col l%16, rows 4*(l/16) + j   (j = 0..3)
//   ds_read_b64_tr_b16: within each 16-lane group, lane i supplies the address of
//     4 consecutive 16-bit elements that form row i/4, columns 4*(i%4)..+3 of a
//     4x16 tile; lane j receives column j of that tile (rows 0..3).
// Because the k index of an MFMA is summed over, any bijection between (lane
// group, element) and the contracted index works as long as both operands use
// the same one; the kernels rely on that to read operands in their natural
// memory order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));

#define ATTN_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 2^x on the transcendental unit (no denormal fix-up; -inf gives 0).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Combine a lane's value with that of lane l ^ 32 (one permlane32 swap).
__device__ __forceinline__ float max_xor32(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Combine with lane l ^ 16 (one permlane16 swap between odd/even 16-lane rows).
__device__ __forceinline__ float max_xor16(float x) {
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Round-to-nearest-even packing of two floats into bf16 (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 r;
  r[0] = (bf16)a;
  r[1] = (bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x4 lds_read_tr(const ATTN_LDS bf16x4* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(const_cast<ATTN_LDS bf16x4*>(p));
}

__device__ __forceinline__ bf16x8 join(const bf16x4& lo, const bf16x4& hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// 16-byte load of data that is read once (global_load_dwordx4 ... nt): the
// caches hold it at streaming priority. For scattered 2-4 KiB block reads this
// draws about 11% more HBM bandwidth than the default policy (measured; for
// the contiguous rows of the append kernel it is slower, so only the paged
// attention kernels use it).
__device__ __forceinline__ u32x4 load_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

constexpr unsigned kRsrcWord3 = 0x00020000u;  // raw (unformatted) buffer descriptor, gfx9

// Buffer descriptor over [base, base + bytes): reads past the end return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kRsrcWord3);
}

// 16 bytes per lane from rsrc + voff into LDS at lds + 16 * lane (lds uniform).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, ATTN_LDS void* lds, unsigned voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, voff, 0, 0, 0);
}

// Wait until at most N vector-memory loads of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0xF70);
}

// Workgroup barrier that orders LDS accesses only (outstanding global loads,
// i.e. the prefetch of later tiles, are not waited for).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Workgroup id after an XCD-aware remap. The dispatcher hands consecutive
// workgroup ids to the 8 XCDs in turn; this gives XCD x the contiguous logical
// range [x * n / 8, (x + 1) * n / 8) so that workgroups sharing K/V (the tiles
// of one head) land on the same XCD and share its L2. Identity when n % 8 != 0.
__device__ __forceinline__ int xcd_remap(int id, int n) {
  if (n % 8 != 0) return id;
  return (id % 8) * (n / 8) + id / 8;
}

}  // namespace attn
