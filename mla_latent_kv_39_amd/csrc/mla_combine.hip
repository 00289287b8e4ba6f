// LSE-merge of the split-KV partials of sequences that mla_decode cut across
// work partitions.  For each such sequence, query token and head:
//     LSE = log sum_s exp(lse_s),   out = sum_s exp(lse_s - LSE) out_s,
// the log-sum-exp identity of one softmax over the union of the partitions'
// rows.
//
// One workgroup merges one quarter of the latent columns (128) of one group
// of 32 heads of one (sequence, query token).  Partials are stored in the
// decode kernel's lane order (see the partial_out layout in include/mla.h):
// the quarter is two contiguous 8 KB runs (head halves a = 0, 1), so thread t
// reads 16-byte chunks t and t + 256 of each run, consecutive threads reading
// consecutive memory, and touches two heads (16a + (t & 15)).  The merged
// quarter goes through LDS once to be written back in row order.
#include "mla_internal.h"
#include "mla_schedule.h"

namespace mla {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kGroupHeads = 32;
constexpr int kQuarterChunks = kGroupHeads * kLatent / 16;   // 16-byte chunks per quarter (1024)
constexpr int kPerThread = kQuarterChunks / 256;             // 4: chunks k = 0, 1 head half 0; 2, 3 head half 1

// LDS slot of lane-order chunk c: XOR the head bits with the column phase so
// that both the lane-order writes and the row-order reads spread over all banks.
__device__ __forceinline__ int lds_slot(int c) { return c ^ ((((c >> 6) & 3) << 2) | ((c >> 4) & 3)); }

__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  __shared__ float4 s_tile[kQuarterChunks];
  __shared__ int s_red[8];
  const int tid = threadIdx.x;
  const int per_tok = (kHeads / kGroupHeads) * 4;
  const int b = blockIdx.x / (p.s_q * per_tok);
  const int s = (blockIdx.x / per_tok) % p.s_q;
  const int grp = (blockIdx.x >> 2) % (kHeads / kGroupHeads);
  const int quarter = blockIdx.x & 3;

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
  const int u1 = u0 + units_of_len(p.seq_lens[b]);
  const int p0 = part_of_unit(u0, total_units, p.num_parts);
  const int p1 = part_of_unit(u1 - 1, total_units, p.num_parts);
  if (p0 == p1) return;  // finished by the decode kernel

  const int r = tid & 15;
  const int head0 = grp * kGroupHeads + r;  // head of chunks k < 2; chunks k >= 2 hold head0 + 16
  // lane-order offset (in chunks) of chunk k inside the group: run a = k >> 1 at 2048 a, quarter at 512 q
  int coff[kPerThread];
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) coff[k] = 2048 * (k >> 1) + 512 * quarter + tid + 256 * (k & 1);
  // pass 1: the largest lse of each of the thread's two heads
  float m[2] = {kNegInf, kNegInf};
  for (int q = p0; q <= p1; ++q) {
    const int q_start = part_start(q, total_units, p.num_parts);
    if (q_start == part_start(q + 1, total_units, p.num_parts)) continue;  // empty partition (more partitions than units)
    const int slot = (q == p0 && u0 != q_start) ? 1 : 0;
    const size_t row = ((size_t)(q * 2 + slot) * p.s_q + s) * kHeads;
    m[0] = fmaxf(m[0], p.part_lse[row + head0]);
    m[1] = fmaxf(m[1], p.part_lse[row + head0 + 16]);
  }
  // pass 2: weighted sums; the loop body has no data-dependent branch, so the
  // loads of successive partitions can be in flight together.  An empty
  // partition reads partition p0's share (always written) with weight 0.
  float wsum[2] = {0.f, 0.f};
  float4 acc[kPerThread];
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) acc[k] = make_float4(0.f, 0.f, 0.f, 0.f);
  const size_t row0 = ((size_t)(p0 * 2 + (u0 != part_start(p0, total_units, p.num_parts) ? 1 : 0)) * p.s_q + s) * kHeads;
#pragma unroll 4
  for (int q = p0; q <= p1; ++q) {
    const int q_start = part_start(q, total_units, p.num_parts);
    const bool empty = q_start == part_start(q + 1, total_units, p.num_parts);
    const int slot = (q == p0 && u0 != q_start) ? 1 : 0;
    const size_t row = empty ? row0 : ((size_t)(q * 2 + slot) * p.s_q + s) * kHeads;
    const float4* src = (const float4*)(p.part_out + (row + grp * kGroupHeads) * kLatent);
    float w[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const float l = p.part_lse[row + head0 + 16 * a];
      // -inf: this share saw no row of this query token
      w[a] = (empty || l == kNegInf) ? 0.f : __expf(l - m[a]);
      wsum[a] += w[a];
    }
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const float wk = w[k >> 1];
      const float4 v = src[coff[k]];
      acc[k].x += wk * v.x; acc[k].y += wk * v.y; acc[k].z += wk * v.z; acc[k].w += wk * v.w;
    }
  }
  float inv[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) inv[a] = wsum[a] > 0.f ? 1.f / wsum[a] : 0.f;
  // quarter-local lane-order chunk: 512 a + 64 (cb - 8 quarter) + lane
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const float ik = inv[k >> 1];
    s_tile[lds_slot(512 * (k >> 1) + tid + 256 * (k & 1))] =
        make_float4(acc[k].x * ik, acc[k].y * ik, acc[k].z * ik, acc[k].w * ik);
  }
  const size_t orow = ((size_t)b * p.s_q + s) * kHeads + grp * kGroupHeads;
  if (tid < 16 && quarter == 0) {
#pragma unroll
    for (int a = 0; a < 2; ++a) p.lse[orow + r + 16 * a] = wsum[a] > 0.f ? m[a] + __logf(wsum[a]) : kNegInf;
  }
  __syncthreads();
  // row order: chunk e of the quarter is head e >> 5, columns 128 quarter + 4 (e & 31) .. +3
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const int e = tid + 256 * k;
    const int hl = e >> 5, cc = e & 31;
    const int c = 512 * (hl >> 4) + 64 * (cc >> 2) + 16 * (cc & 3) + (hl & 15);
    float4* dst = (float4*)(p.out + (orow + hl) * kLatent + 128 * quarter) + cc;
    *dst = s_tile[lds_slot(c)];
  }
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
  const int blocks = p.batch * p.s_q * (kHeads / kGroupHeads) * 4;
  combine_kernel<<<dim3(blocks), dim3(256), 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace mla
