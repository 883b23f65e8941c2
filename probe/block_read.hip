// Read-bandwidth probe: what HBM delivers for a given block access pattern.
// A measurement aid of the benchmark, built into its own library
// (libattn_probe.so); the attention library does not contain it.
//
// The paged kernels read the cache as scattered (block, head) slabs of 2 or 4
// KiB; the ceiling of such a kernel is the rate HBM sustains for that pattern,
// not the 8 TB/s of streaming reads (the roofline argument of [P4]: a
// memory-bound kernel is measured against the bandwidth its accesses can draw).
// This kernel does nothing but those reads: each wave takes whole blocks from
// an order list, two blocks in flight, 16 bytes per lane per load (with the
// default or the nontemporal cache policy), and folds every word into a
// per-lane XOR that it stores at the end, so that no load is dead and the
// result can be checked.
#include "../attention_tiled_qk_amd/csrc/common.h"

namespace attn {

template <bool NT>
__device__ __forceinline__ u32x4 probe_load(const u32x4* p) {
  if constexpr (NT) return load_stream(p);
  else return *p;
}

template <int CH, bool NT>  // 1 KiB chunks per block; nontemporal loads
__global__ __launch_bounds__(256) void block_read_kernel(const u32x4* __restrict__ buf,
                                                         const int32_t* __restrict__ order,
                                                         int n_reads, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int n_waves = gridDim.x * 4;
  u32x4 acc = {0u, 0u, 0u, 0u};
  int i = wave;
  for (; i + n_waves < n_reads; i += 2 * n_waves) {
    const u32x4* a = buf + (size_t)order[i] * CH * 64;
    const u32x4* b = buf + (size_t)order[i + n_waves] * CH * 64;
    u32x4 va[CH], vb[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) va[c] = probe_load<NT>(a + c * 64 + lane);
#pragma unroll
    for (int c = 0; c < CH; ++c) vb[c] = probe_load<NT>(b + c * 64 + lane);
#pragma unroll
    for (int c = 0; c < CH; ++c) acc ^= va[c] ^ vb[c];
  }
  if (i < n_reads) {
    const u32x4* a = buf + (size_t)order[i] * CH * 64;
#pragma unroll
    for (int c = 0; c < CH; ++c) acc ^= probe_load<NT>(a + c * 64 + lane);
  }
  sink[(size_t)wave * 64 + lane] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

template <bool NT>
static void launch_probe_variant(const u32x4* p, int block_bytes, const int32_t* order, int n_reads,
                                 uint32_t* sink, dim3 grid, hipStream_t stream) {
  const dim3 block(256);
  switch (block_bytes / 1024) {
    case 1:
      hipLaunchKernelGGL((block_read_kernel<1, NT>), grid, block, 0, stream, p, order, n_reads, sink);
      break;
    case 2:
      hipLaunchKernelGGL((block_read_kernel<2, NT>), grid, block, 0, stream, p, order, n_reads, sink);
      break;
    case 4:
      hipLaunchKernelGGL((block_read_kernel<4, NT>), grid, block, 0, stream, p, order, n_reads, sink);
      break;
    case 8:
      hipLaunchKernelGGL((block_read_kernel<8, NT>), grid, block, 0, stream, p, order, n_reads, sink);
      break;
    default:
      hipLaunchKernelGGL((block_read_kernel<16, NT>), grid, block, 0, stream, p, order, n_reads, sink);
      break;
  }
}

}  // namespace attn

extern "C" {

// Reads the blocks order[0 .. n_reads) of buf (num_blocks blocks of
// block_bytes, 16-byte aligned) and nothing else; lane l of wave w stores the
// XOR of the 32-bit words it read in sink[w * 64 + l], so the XOR of all sink
// words equals the XOR of every word of every block read. Wave w reads
// order[w], order[w + n_waves], ..., two blocks at a time. block_bytes: 1, 2,
// 4, 8 or 16 KiB; n_waves a multiple of 4 in [4, 2^22]; nontemporal 0 or 1
// selects the cache policy of the loads. Ids are not checked on the device.
// Returns 0, or -2 (bad size), -4 (unsupported block size), -5 (misaligned),
// -1 (null pointer), -8 (launch failed); nothing is enqueued on error.
int probe_block_read(const void* buf, int num_blocks, int block_bytes, const int32_t* order,
                     int n_reads, uint32_t* sink, int n_waves, int nontemporal, void* stream) {
  using namespace attn;
  if (!buf || !order || !sink) return -1;
  if (num_blocks <= 0 || n_reads <= 0) return -2;
  if (block_bytes != 1024 && block_bytes != 2048 && block_bytes != 4096 && block_bytes != 8192 &&
      block_bytes != 16384)
    return -4;
  if (n_waves < 4 || n_waves > (1 << 22) || n_waves % 4 != 0) return -2;
  if (nontemporal != 0 && nontemporal != 1) return -2;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0) return -5;
  if ((reinterpret_cast<uintptr_t>(order) & 3u) != 0 || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0)
    return -5;
  const u32x4* p = static_cast<const u32x4*>(buf);
  const dim3 grid(n_waves / 4);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (nontemporal) launch_probe_variant<true>(p, block_bytes, order, n_reads, sink, grid, s);
  else launch_probe_variant<false>(p, block_bytes, order, n_reads, sink, grid, s);
  return hipGetLastError() == hipSuccess ? 0 : -8;
}

}  // extern "C"
