// The index contract of the decode, checked on the device: every sequence
// length lies in [0, max_blocks * 64] and every block-table entry of a page a
// sequence uses names a page of the cache.  One workgroup walks all lengths
// and all (sequence, page) pairs and writes the two counts (no atomics, no
// pre-cleared memory: the counts are plain stores of the workgroup's sums).
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kThreads = 1024;

__global__ __launch_bounds__(kThreads) void check_indices_kernel(CheckParams p) {
  __shared__ int s_sum[2][kThreads / 64];
  const int tid = threadIdx.x;
  const long long cap = (long long)p.max_blocks * kPage;
  int bad_len = 0, bad_entry = 0;
  for (int b = tid; b < p.batch; b += kThreads) {
    const int len = p.seq_lens[b];
    bad_len += (len < 0 || (long long)len > cap) ? 1 : 0;
  }
  const long long pairs = (long long)p.batch * p.max_blocks;
  for (long long i = tid; i < pairs; i += kThreads) {
    const int b = (int)(i / p.max_blocks);
    const int u = (int)(i - (long long)b * p.max_blocks);
    const int len = p.seq_lens[b];
    const int used = len > 0 ? (len + kPage - 1) / kPage : 0;
    if (u < used) {
      const long long page = p.block_table ? (long long)p.block_table[i] : i;
      bad_entry += (page < 0 || page >= p.num_blocks) ? 1 : 0;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    bad_len += __shfl_xor(bad_len, off);
    bad_entry += __shfl_xor(bad_entry, off);
  }
  if ((tid & 63) == 0) {
    s_sum[0][tid >> 6] = bad_len;
    s_sum[1][tid >> 6] = bad_entry;
  }
  __syncthreads();
  if (tid == 0) {
    int a = 0, c = 0;
    for (int w = 0; w < kThreads / 64; ++w) {
      a += s_sum[0][w];
      c += s_sum[1][w];
    }
    p.counts[0] = a;
    p.counts[1] = c;
  }
}

}  // namespace

hipError_t launch_check_indices(const CheckParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(check_indices_kernel, dim3(1), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
