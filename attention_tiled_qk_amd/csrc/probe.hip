// Read-bandwidth probe: what HBM delivers for a given block access pattern.
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
#include "common.h"

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

hipError_t launch_probe_block_read(const void* buf, int block_bytes, const int32_t* order,
                                   int n_reads, uint32_t* sink, int n_waves, int nontemporal,
                                   hipStream_t stream) {
  const u32x4* p = static_cast<const u32x4*>(buf);
  const dim3 grid(n_waves / 4);
  if (nontemporal) launch_probe_variant<true>(p, block_bytes, order, n_reads, sink, grid, stream);
  else launch_probe_variant<false>(p, block_bytes, order, n_reads, sink, grid, stream);
  return hipGetLastError();
}

}  // namespace attn
