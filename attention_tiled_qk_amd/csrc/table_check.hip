// Validation of a paged-cache description (block tables and sequence lengths).
//
// The attention, append and gather kernels trust their tables: a request's
// table lists the only blocks its kernel reads ([P3] PagedAttention item), so
// an id outside the pool or a length past the table's width would make them
// read or write memory that belongs to no block. This kernel only reads the
// tables and counts such entries, as a debugging aid to run before those calls.
#include "common.h"

namespace attn {

constexpr int kCheckThreads = 256;

// One workgroup walks every sequence, so the two counts need no atomics and no
// zeroed output: each thread counts its share, the workgroup adds the shares
// in LDS and thread 0 writes the totals, saturated at INT32_MAX.
__global__ __launch_bounds__(kCheckThreads) void check_tables_kernel(
    const int32_t* __restrict__ tables, const int32_t* __restrict__ lens, int B, int min_len,
    int num_blocks, int width, int32_t* __restrict__ bad) {
  __shared__ long long red[2][kCheckThreads];
  const int tid = threadIdx.x;
  long long bad_len = 0, bad_id = 0;
  const long long cap = 16LL * width;  // keys the table can address
  for (int b = 0; b < B; ++b) {
    const long long n = lens[b];
    if (tid == 0 && (n < min_len || n > cap)) ++bad_len;
    const int nb = (int)((max(0LL, min(n, cap)) + 15) / 16);  // entries the calls read
    const int32_t* row = tables + (size_t)b * width;
    for (int j = tid; j < nb; j += kCheckThreads) {
      const int id = row[j];
      bad_id += (id < 0 || id >= num_blocks) ? 1 : 0;
    }
  }
  red[0][tid] = bad_len;
  red[1][tid] = bad_id;
  __syncthreads();
  for (int s = kCheckThreads / 2; s > 0; s >>= 1) {
    if (tid < s) {
      red[0][tid] += red[0][tid + s];
      red[1][tid] += red[1][tid + s];
    }
    __syncthreads();
  }
  if (tid == 0) {
    bad[0] = (int32_t)min(red[0][0], (long long)INT32_MAX);
    bad[1] = (int32_t)min(red[1][0], (long long)INT32_MAX);
  }
}

hipError_t launch_check_tables(const int32_t* tables, const int32_t* lens, int B, int min_len,
                               int num_blocks, int width, int32_t* bad, hipStream_t stream) {
  hipLaunchKernelGGL(check_tables_kernel, dim3(1), dim3(kCheckThreads), 0, stream, tables, lens, B,
                     min_len, num_blocks, width, bad);
  return hipGetLastError();
}

}  // namespace attn
