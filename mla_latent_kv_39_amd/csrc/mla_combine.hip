// LSE-merge of the split-KV partials of sequences that mla_decode cut across
// work partitions.  For each such sequence, query token and head:
//     LSE = log sum_s exp(lse_s),   out = sum_s exp(lse_s - LSE) out_s,
// the log-sum-exp identity of one softmax over the union of the partitions'
// rows.  One workgroup handles 16 heads x 512 latent values of one
// (sequence, query token); each thread owns 32 consecutive values of one head.
#include "mla_internal.h"
#include "mla_schedule.h"

namespace mla {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();

__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  __shared__ int s_scan[256];
  const int tid = threadIdx.x;
  const int per_seq = p.s_q * (kHeads / 16);
  const int b = blockIdx.x / per_seq;
  const int s = (blockIdx.x / (kHeads / 16)) % p.s_q;
  const int hg = blockIdx.x % (kHeads / 16);

  // rebuild the partition map: total units and the first unit of sequence b
  const int B = p.batch;
  const int per = (B + 255) >> 8;
  const int b_lo = min(B, tid * per), b_hi = min(B, b_lo + per);
  int cnt = 0, before = 0;
  for (int i = b_lo; i < b_hi; ++i) {
    const int n = units_of_len(p.seq_lens[i]);
    cnt += n;
    if (i < b) before += n;
  }
  int total_units, u0;
  block_exclusive_scan_256(cnt, s_scan, &total_units);
  block_exclusive_scan_256(before, s_scan, &u0);
  const int u1 = u0 + units_of_len(p.seq_lens[b]);
  const int p0 = part_of_unit(u0, total_units, p.num_parts);
  const int p1 = part_of_unit(u1 - 1, total_units, p.num_parts);
  if (p0 == p1) return;  // finished by the decode kernel

  const int head = hg * 16 + (tid >> 4);
  const int col = (tid & 15) * 32;
  float m = kNegInf, wsum = 0.f;
  float acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = 0.f;
  for (int q = p0; q <= p1; ++q) {
    const int q_start = part_start(q, total_units, p.num_parts);
    if (q_start == part_start(q + 1, total_units, p.num_parts)) continue;  // empty partition (more partitions than units)
    const int slot = (q == p0 && u0 != q_start) ? 1 : 0;
    const size_t ridx = ((size_t)(q * 2 + slot) * p.s_q + s) * kHeads + head;
    const float l = p.part_lse[ridx];
    if (l == kNegInf) continue;  // this share saw no row of this query token
    const float4* src = (const float4*)(p.part_out + ridx * kLatent + col);
    float w;
    if (l > m) {
      const float r = __expf(m - l);
      wsum *= r;
#pragma unroll
      for (int i = 0; i < 32; ++i) acc[i] *= r;
      m = l;
      w = 1.f;
    } else {
      w = __expf(l - m);
    }
    wsum += w;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 v = src[i];
      acc[4 * i + 0] += w * v.x;
      acc[4 * i + 1] += w * v.y;
      acc[4 * i + 2] += w * v.z;
      acc[4 * i + 3] += w * v.w;
    }
  }
  const size_t oidx = ((size_t)b * p.s_q + s) * kHeads + head;
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  float4* dst = (float4*)(p.out + oidx * kLatent + col);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    dst[i] = make_float4(acc[4 * i] * inv, acc[4 * i + 1] * inv, acc[4 * i + 2] * inv, acc[4 * i + 3] * inv);
  if ((tid & 15) == 0) p.lse[oidx] = wsum > 0.f ? m + __logf(wsum) : kNegInf;
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
  const int blocks = p.batch * p.s_q * (kHeads / 16);
  combine_kernel<<<dim3(blocks), dim3(256), 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace mla
