// LSE-merge of the split-KV partials of sequences that mla_decode cut across
// work partitions.  For each such sequence, query token and head:
//     LSE = log sum_s exp(lse_s),   out = sum_s exp(lse_s - LSE) out_s,
// the log-sum-exp identity of one softmax over the union of the partitions'
// rows.
//
// One workgroup merges one slice of the latent columns (16 CB of them, CB = 8,
// 4 or 2 column blocks; the host picks the widest slice that still gives
// the GPU enough workgroups) of one group of 32 heads of one (sequence, query
// token).  Partials are stored in the decode kernel's lane order (see the
// partial_out layout in include/mla.h): a slice is two contiguous runs of
// CB KB (head halves a = 0, 1), so consecutive threads read consecutive
// 16-byte chunks.  Partitions are taken in chunks whose loads are all issued
// before any is used, each chunk merged into a running (max, sum, accumulator)
// triple, so a sequence cut into few partitions costs one memory round trip.
// The merged slice goes through LDS once to be written back in row order.
#include "mla_internal.h"
#include "mla_schedule.h"

namespace mla {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kGroupHeads = 32;

// LDS slot of lane-order chunk c: XOR the head bits with the column phase so
// that both the lane-order writes and the row-order reads spread over all banks.
__device__ __forceinline__ int lds_slot(int c) { return c ^ ((((c >> 6) & 3) << 2) | ((c >> 4) & 3)); }

template <int CB>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  constexpr int kSlices = 32 / CB;
  constexpr int kRun = 64 * CB;                // chunks per head half of a slice
  constexpr int kPerThread = 2 * kRun / 256;   // 4, 2 or 1
  constexpr int kChunk = 4;                    // partitions whose loads are in flight together
  __shared__ float4 s_tile[2 * kRun];
  __shared__ int s_red[8];
  const int tid = threadIdx.x;
  const int per_tok = (kHeads / kGroupHeads) * kSlices;
  const int b = blockIdx.x / (p.s_q * per_tok);
  const int s = (blockIdx.x / per_tok) % p.s_q;
  const int grp = (blockIdx.x / kSlices) % (kHeads / kGroupHeads);
  const int slice = blockIdx.x % kSlices;

  // rebuild the partition map: total units U and the first unit u0 of sequence b
  int cnt = 0, before = 0;
  for (int i = tid; i < p.batch; i += 256) {
    const int n = units_of_len(p.seq_lens[i]);
    cnt += n;
    if (i < b) before += n;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    cnt += __shfl_xor(cnt, off);
    before += __shfl_xor(before, off);
  }
  if ((tid & 63) == 0) {
    s_red[2 * (tid >> 6)] = cnt;
    s_red[2 * (tid >> 6) + 1] = before;
  }
  __syncthreads();
  const int total_units = s_red[0] + s_red[2] + s_red[4] + s_red[6];
  const int u0 = s_red[1] + s_red[3] + s_red[5] + s_red[7];
  const int nb = units_of_len(p.seq_lens[b]);
  const int weight = total_units + p.batch * kSegWeight;
  // weighted positions of the sequence's first and last units
  const int x0 = u0 + (b + 1) * kSegWeight;
  const int x1 = x0 + nb - 1;
  const int p0 = part_of_pos(x0, weight, p.num_parts);
  const int p1 = part_of_pos(x1, weight, p.num_parts);
  if (p0 == p1) return;  // finished by the decode kernel
  // partition p0 also holds units of the sequence before (it ends in this one:
  // slot 1) iff that sequence's last unit lies at or past its start
  const int slot0 = (b > 0 && u0 - 1 + b * kSegWeight >= part_start(p0, weight, p.log2_parts)) ? 1 : 0;

  // chunk k of this thread: slice-local index t + 256 k, head half a, lane-order offset in the group
  int head[kPerThread], coff[kPerThread];
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const int lc = tid + 256 * k;
    const int a = lc / kRun;
    head[k] = grp * kGroupHeads + 16 * a + (tid & 15);
    coff[k] = 2048 * a + kRun * slice + lc % kRun;
  }
  float m[kPerThread], wsum[kPerThread];
  float4 acc[kPerThread];
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    m[k] = kNegInf;
    wsum[k] = 0.f;
    acc[k] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  // partitions in chunks of kChunk: all loads of a chunk go out before any is
  // used (one memory round trip per chunk), then the chunk is merged into the
  // running (m, wsum, acc) with a rescale when its largest lse is new
  for (int qb = p0; qb <= p1; qb += kChunk) {
    float l[kChunk][kPerThread];
    float4 v[kChunk][kPerThread];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      const int q = qb + i;
      // a partition past the sequence or without units holds no share
      const bool live = q <= p1 && part_start(q, weight, p.log2_parts) != part_start(q + 1, weight, p.log2_parts);
      const size_t row = ((size_t)(q * 2 + (q == p0 ? slot0 : 0)) * p.s_q + s) * kHeads;
      const float4* src = (const float4*)(p.part_out + (row + grp * kGroupHeads) * kLatent);
#pragma unroll
      for (int k = 0; k < kPerThread; ++k) {
        l[i][k] = kNegInf;
        v[i][k] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (live) {
          l[i][k] = p.part_lse[row + head[k]];     // -inf: the share saw no row of this token
          v[i][k] = src[coff[k]];
        }
      }
    }
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      float mc = m[k];
#pragma unroll
      for (int i = 0; i < kChunk; ++i) mc = fmaxf(mc, l[i][k]);
      if (mc == kNegInf) continue;          // nothing seen yet
      const float r = __expf(m[k] - mc);    // 0 while m is -inf
      wsum[k] *= r;
      acc[k].x *= r; acc[k].y *= r; acc[k].z *= r; acc[k].w *= r;
      m[k] = mc;
#pragma unroll
      for (int i = 0; i < kChunk; ++i) {
        const float w = __expf(l[i][k] - mc);   // 0 for -inf
        wsum[k] += w;
        acc[k].x += w * v[i][k].x; acc[k].y += w * v[i][k].y; acc[k].z += w * v[i][k].z; acc[k].w += w * v[i][k].w;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const float ik = wsum[k] > 0.f ? 1.f / wsum[k] : 0.f;
    s_tile[lds_slot(tid + 256 * k)] = make_float4(acc[k].x * ik, acc[k].y * ik, acc[k].z * ik, acc[k].w * ik);
  }
  const size_t orow = ((size_t)b * p.s_q + s) * kHeads + grp * kGroupHeads;
  if (slice == 0) {
    // lse of the group's heads: the threads whose chunk k sits in column block 0, g == 0
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const int lc = tid + 256 * k;
      if ((lc % kRun) < 16) p.lse[head[k]  - grp * kGroupHeads + orow] = wsum[k] > 0.f ? m[k] + __logf(wsum[k]) : kNegInf;
    }
  }
  __syncthreads();
  // row order: chunk e of the slice is head e / (4 CB), columns 16 CB slice + 4 (e % (4 CB)) .. +3
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const int e = tid + 256 * k;
    const int hl = e / (4 * CB), cc = e % (4 * CB);
    const int c = kRun * (hl >> 4) + 64 * (cc >> 2) + 16 * (cc & 3) + (hl & 15);
    float4* dst = (float4*)(p.out + (orow + hl) * kLatent + 16 * CB * slice) + cc;
    *dst = s_tile[lds_slot(c)];
  }
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
  // widest column slice that still gives about eight workgroups per compute
  // unit: the shares of short and long sequences then mix on every unit
  const long long base = (long long)p.batch * p.s_q * (kHeads / kGroupHeads);
  const long long want = 2048;
  if (base * 4 >= want) {
    combine_kernel<8><<<dim3((unsigned)(base * 4)), dim3(256), 0, stream>>>(p);
  } else if (base * 8 >= want) {
    combine_kernel<4><<<dim3((unsigned)(base * 8)), dim3(256), 0, stream>>>(p);
  } else {
    combine_kernel<2><<<dim3((unsigned)(base * 16)), dim3(256), 0, stream>>>(p);
  }
  return hipGetLastError();
}

}  // namespace mla
