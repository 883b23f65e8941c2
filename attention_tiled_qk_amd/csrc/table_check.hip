// Validation of a paged-cache description (block tables, sequence lengths,
// packed query offsets, block-id lists).
//
// The attention, append, gather and copy kernels trust their device arrays: a
// request's table lists the only blocks its kernel reads ([P3] PagedAttention
// item), so an id outside the pool, a length past the table's width or a query
// offset past the packed tensor would make them read or write memory that
// belongs to no block or no row. The kernels here only read those arrays and
// count such entries, as debugging aids to run before the calls.
#include "common.h"

namespace attn {

constexpr int kCheckThreads = 256;

// Adds the per-thread counts of the workgroup and has thread 0 write them,
// saturated at INT32_MAX, so no atomics and no zeroed output are needed.
__device__ void write_counts(long long c0, long long c1, int32_t* __restrict__ bad) {
  __shared__ long long red[2][kCheckThreads];
  const int tid = threadIdx.x;
  red[0][tid] = c0;
  red[1][tid] = c1;
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

// Attention and gather calls: lengths in [min_len, 16 * width]; the entries a
// call reads (the first ceil(len / 16) of a row) inside [0, num_blocks).
__global__ __launch_bounds__(kCheckThreads) void check_tables_kernel(
    const int32_t* __restrict__ tables, const int32_t* __restrict__ lens, int B, int min_len,
    int num_blocks, int width, int32_t* __restrict__ bad) {
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
  write_counts(bad_len, bad_id, bad);
}

// Append calls: lengths in [0, 16 * width]; the entries covering the n_new
// newest positions (those >= 0) are -1 (nothing is placed there) or inside
// [0, num_blocks). This is the rule the append kernels apply.
__global__ __launch_bounds__(kCheckThreads) void check_append_kernel(
    const int32_t* __restrict__ tables, const int32_t* __restrict__ lens, int B, int n_new,
    int num_blocks, int width, int32_t* __restrict__ bad) {
  const int tid = threadIdx.x;
  long long bad_len = 0, bad_id = 0;
  const long long cap = 16LL * width;
  for (int b = 0; b < B; ++b) {
    const long long n = lens[b];
    if (tid == 0 && (n < 0 || n > cap)) ++bad_len;
    const long long hi = min(n, cap);  // one past the newest position written
    const long long lo = max(0LL, hi - n_new);
    if (hi <= lo) continue;
    const int first = (int)(lo / 16), last = (int)((hi - 1) / 16);
    const int32_t* row = tables + (size_t)b * width;
    for (int j = first + tid; j <= last; j += kCheckThreads) {
      const int id = row[j];
      bad_id += (id < -1 || id >= num_blocks) ? 1 : 0;
    }
  }
  write_counts(bad_len, bad_id, bad);
}

// Ragged prefill calls: bad[0] counts offset errors (cu[0] != 0, cu[B] !=
// total_q, a decreasing step); bad[1] counts sequences whose query count
// exceeds max_q_len or its own length seq_lens[b].
__global__ __launch_bounds__(kCheckThreads) void check_ragged_kernel(
    const int32_t* __restrict__ cu, const int32_t* __restrict__ lens, int B, int total_q,
    int max_q_len, int32_t* __restrict__ bad) {
  const int tid = threadIdx.x;
  long long bad_off = 0, bad_seq = 0;
  if (tid == 0) bad_off += (cu[0] != 0) + (cu[B] != total_q);
  for (int b = tid; b < B; b += kCheckThreads) {
    const long long n = (long long)cu[b + 1] - cu[b];
    if (n < 0) ++bad_off;
    else if (n > max_q_len || n > lens[b]) ++bad_seq;
  }
  write_counts(bad_off, bad_seq, bad);
}

// Block-id lists (the copy calls): bad[0] counts entries of src and bad[1]
// entries of dst outside [0, num_blocks).
__global__ __launch_bounds__(kCheckThreads) void check_ids_kernel(
    const int32_t* __restrict__ src, const int32_t* __restrict__ dst, int n, int num_blocks,
    int32_t* __restrict__ bad) {
  long long bs = 0, bd = 0;
  for (int i = threadIdx.x; i < n; i += kCheckThreads) {
    bs += (src[i] < 0 || src[i] >= num_blocks) ? 1 : 0;
    bd += (dst[i] < 0 || dst[i] >= num_blocks) ? 1 : 0;
  }
  write_counts(bs, bd, bad);
}

hipError_t launch_check_tables(const int32_t* tables, const int32_t* lens, int B, int min_len,
                               int num_blocks, int width, int32_t* bad, hipStream_t stream) {
  hipLaunchKernelGGL(check_tables_kernel, dim3(1), dim3(kCheckThreads), 0, stream, tables, lens, B,
                     min_len, num_blocks, width, bad);
  return hipGetLastError();
}

hipError_t launch_check_append(const int32_t* tables, const int32_t* lens, int B, int n_new,
                               int num_blocks, int width, int32_t* bad, hipStream_t stream) {
  hipLaunchKernelGGL(check_append_kernel, dim3(1), dim3(kCheckThreads), 0, stream, tables, lens, B,
                     n_new, num_blocks, width, bad);
  return hipGetLastError();
}

hipError_t launch_check_ragged(const int32_t* cu, const int32_t* lens, int B, int total_q,
                               int max_q_len, int32_t* bad, hipStream_t stream) {
  hipLaunchKernelGGL(check_ragged_kernel, dim3(1), dim3(kCheckThreads), 0, stream, cu, lens, B,
                     total_q, max_q_len, bad);
  return hipGetLastError();
}

hipError_t launch_check_ids(const int32_t* src, const int32_t* dst, int n, int num_blocks,
                            int32_t* bad, hipStream_t stream) {
  hipLaunchKernelGGL(check_ids_kernel, dim3(1), dim3(kCheckThreads), 0, stream, src, dst, n,
                     num_blocks, bad);
  return hipGetLastError();
}

}  // namespace attn
