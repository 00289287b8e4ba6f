// LSE-merge of the split-KV partials of sequences that mla_decode cut across
// work partitions.  For each such sequence, query token and head:
//     LSE = log sum_s exp(lse_s),   out = sum_s exp(lse_s - LSE) out_s,
// the log-sum-exp identity of one softmax over the union of the partitions'
// rows.
//
// One workgroup merges one slice of the latent columns (16 CB of them, CB = 8,
// 4 or 2 column blocks; the host picks the widest slice that still gives the
// GPU enough workgroups) of one group of 32 heads of one (sequence, query
// token).  Partials are fp16 in the decode kernels' lane order with one
// power-of-two descale per (block, column quarter, head) (the partial_out
// layout in include/mla.h): a slice is one contiguous run of CB KB, 16-byte
// chunks of two heads (r, r + 16) x four columns, so consecutive threads read
// consecutive chunks.  Partitions are taken in chunks (4, or 8-16 when
// sequences are cut into many) whose loads are all issued before any is
// used, each chunk merged into a running (max, sum, accumulator) triple per
// head, so a sequence cut into few partitions costs one memory round trip.
// The merged slice goes through LDS once to be written back in row order.
#include <hip/hip_fp16.h>

#include "mla_internal.h"
#include "mla_schedule.h"

namespace mla {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kGroupHeads = 32;

// LDS slot of a (head half, column block, lane) float4 c: XOR the head bits with
// the column phase so that both the lane-order writes and the row-order reads
// spread over all banks.
__device__ __forceinline__ int lds_slot(int c) { return c ^ ((((c >> 6) & 3) << 2) | ((c >> 4) & 3)); }

__device__ __forceinline__ float4 half4(uint2 h) {
  const __half2 a = *reinterpret_cast<const __half2*>(&h.x);
  const __half2 b = *reinterpret_cast<const __half2*>(&h.y);
  return make_float4(__low2float(a), __high2float(a), __low2float(b), __high2float(b));
}

// TS > 1: TS groups of threads share a sequence's partitions (group g takes
// chunks g, g + TS, ...) and their (max, sum, accumulator) triples are then
// merged through LDS in group order, so that a sequence cut into many
// partitions keeps TS times the waves loading.
template <int CB, int KC, int TS>
__global__ __launch_bounds__((CB * 64 < 256 ? CB * 64 : 256) * TS) void combine_kernel(CombineParams p) {
  constexpr int kThreads = CB * 64 < 256 ? CB * 64 : 256;   // one group
  constexpr int kBlock = kThreads * TS;
  constexpr int kSlices = 32 / CB;
  constexpr int kRun = 64 * CB;                 // 16-byte chunks of a slice
  constexpr int kPerThread = kRun / kThreads;   // 2 or 1
  constexpr int kChunk = KC;                    // partitions whose loads are in flight together
  constexpr int kShared = TS > 1 ? (TS - 1) * kPerThread * 2 * kThreads : 1;   // no LDS for one group
  __shared__ float4 s_tile[2 * kRun];
  __shared__ int s_red[2 * (kBlock / 64)];
  __shared__ float s_gm[kShared], s_gw[kShared];
  __shared__ float4 s_ga[kShared];
  // one group: constants, so that the kernel is the plain one (a group index
  // computed at run time cost the paged mix's merge 18%)
  const int tid = TS == 1 ? (int)threadIdx.x : (int)threadIdx.x % kThreads;
  const int sub = TS == 1 ? 0 : (int)threadIdx.x / kThreads;
  const int per_tok = (kHeads / kGroupHeads) * kSlices;
  const int b = blockIdx.x / (p.s_q * per_tok);
  const int s = (blockIdx.x / per_tok) % p.s_q;
  const int grp = (blockIdx.x / kSlices) % (kHeads / kGroupHeads);
  const int slice = blockIdx.x % kSlices;

  // rebuild the partition map: total units U and the first unit u0 of sequence b
  int cnt = 0, before = 0;
  for (int i = (int)threadIdx.x; i < p.batch; i += kBlock) {
    const int n = units_of_len(p.seq_lens[i]);
    cnt += n;
    if (i < b) before += n;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    cnt += __shfl_xor(cnt, off);
    before += __shfl_xor(before, off);
  }
  if ((threadIdx.x & 63) == 0) {
    s_red[2 * (threadIdx.x >> 6)] = cnt;
    s_red[2 * (threadIdx.x >> 6) + 1] = before;
  }
  __syncthreads();
  int total_units = 0, u0 = 0;
#pragma unroll
  for (int w = 0; w < kBlock / 64; ++w) {
    total_units += s_red[2 * w];
    u0 += s_red[2 * w + 1];
  }
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

  // chunk k of this thread: slice-local index tid + kThreads k = 64 cl + 16 g + r,
  // heads grp * 32 + r and + 16, column quarter of the slice
  const int quarter = (CB * slice) >> 3;
  int cidx[kPerThread], r16[kPerThread];
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const int lc = tid + kThreads * k;
    r16[k] = lc & 15;
    cidx[k] = kRun * slice + lc;
  }
  const size_t nblocks = (size_t)p.num_parts * 2 * p.s_q;
  const char* vals = static_cast<const char*>(p.part_out);
  const float* desc = reinterpret_cast<const float*>(vals + nblocks * kPartBlockBytes);
  float m[kPerThread][2], wsum[kPerThread][2];
  float4 acc[kPerThread][2];
#pragma unroll
  for (int k = 0; k < kPerThread; ++k)
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      m[k][a] = kNegInf;
      wsum[k][a] = 0.f;
      acc[k][a] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  // partitions in chunks of kChunk: all loads of a chunk go out before any is
  // used (one memory round trip per chunk), then the chunk is merged into the
  // running (m, wsum, acc) with a rescale when its largest lse is new
  for (int qb = p0 + sub * kChunk; qb <= p1; qb += TS * kChunk) {
    float l[kChunk][kPerThread][2];
    float2 d[kChunk][kPerThread];
    uint4 v[kChunk][kPerThread];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      const int q = qb + i;
      // a partition past the sequence or without units holds no share
      const bool live = q <= p1 && part_start(q, weight, p.log2_parts) != part_start(q + 1, weight, p.log2_parts);
      const size_t blk = (size_t)(q * 2 + (q == p0 ? slot0 : 0)) * p.s_q + s;
      const uint4* src = reinterpret_cast<const uint4*>(vals + blk * kPartBlockBytes) + grp * 2048;
      const float2* dsc = reinterpret_cast<const float2*>(desc + blk * 512 + 128 * quarter + 32 * grp);
      const float* lsrc = p.part_lse + blk * kHeads + grp * kGroupHeads;
#pragma unroll
      for (int k = 0; k < kPerThread; ++k) {
        l[i][k][0] = l[i][k][1] = kNegInf;
        d[i][k] = make_float2(0.f, 0.f);
        v[i][k] = make_uint4(0, 0, 0, 0);
        if (live) {
          l[i][k][0] = lsrc[r16[k]];             // -inf: the share saw no row of this token
          l[i][k][1] = lsrc[r16[k] + 16];
          d[i][k] = dsc[r16[k]];
          v[i][k] = src[cidx[k]];
        }
      }
    }
#pragma unroll
    for (int k = 0; k < kPerThread; ++k)
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        float mc = m[k][a];
#pragma unroll
        for (int i = 0; i < kChunk; ++i) mc = fmaxf(mc, l[i][k][a]);
        if (mc == kNegInf) continue;          // nothing seen yet
        const float r = __expf(m[k][a] - mc);  // 0 while m is -inf
        wsum[k][a] *= r;
        acc[k][a].x *= r; acc[k][a].y *= r; acc[k][a].z *= r; acc[k][a].w *= r;
        m[k][a] = mc;
#pragma unroll
        for (int i = 0; i < kChunk; ++i) {
          const float w = __expf(l[i][k][a] - mc);   // 0 for -inf
          wsum[k][a] += w;
          const float wd = w * (a ? d[i][k].y : d[i][k].x);
          const float4 x = half4(a ? make_uint2(v[i][k].z, v[i][k].w) : make_uint2(v[i][k].x, v[i][k].y));
          acc[k][a].x += wd * x.x; acc[k][a].y += wd * x.y; acc[k][a].z += wd * x.z; acc[k][a].w += wd * x.w;
        }
      }
  }
  if constexpr (TS > 1) {
    // groups 1 .. TS - 1 hand their triples to group 0, which merges them in order
    if (sub > 0) {
#pragma unroll
      for (int k = 0; k < kPerThread; ++k)
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const int x = (((sub - 1) * kPerThread + k) * 2 + a) * kThreads + tid;
          s_gm[x] = m[k][a];
          s_gw[x] = wsum[k][a];
          s_ga[x] = acc[k][a];
        }
    }
    __syncthreads();
    // every thread goes on to the barrier below; only group 0 merges and writes
#pragma unroll
    for (int g = 1; g < (sub == 0 ? TS : 1); ++g)
#pragma unroll
      for (int k = 0; k < kPerThread; ++k)
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const int x = (((g - 1) * kPerThread + k) * 2 + a) * kThreads + tid;
          const float mg = s_gm[x], mc = fmaxf(m[k][a], mg);
          if (mc == kNegInf) continue;
          const float r = __expf(m[k][a] - mc), rg = __expf(mg - mc);   // 0 for -inf
          const float4 ag = s_ga[x];
          wsum[k][a] = wsum[k][a] * r + s_gw[x] * rg;
          acc[k][a].x = acc[k][a].x * r + ag.x * rg;
          acc[k][a].y = acc[k][a].y * r + ag.y * rg;
          acc[k][a].z = acc[k][a].z * r + ag.z * rg;
          acc[k][a].w = acc[k][a].w * r + ag.w * rg;
          m[k][a] = mc;
        }
  }
  const size_t orow = ((size_t)b * p.s_q + s) * kHeads + grp * kGroupHeads;
  if (sub == 0) {
#pragma unroll
    for (int k = 0; k < kPerThread; ++k)
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const float ik = wsum[k][a] > 0.f ? 1.f / wsum[k][a] : 0.f;
        s_tile[lds_slot(kRun * a + tid + kThreads * k)] =
            make_float4(acc[k][a].x * ik, acc[k][a].y * ik, acc[k][a].z * ik, acc[k][a].w * ik);
      }
  }
  if (sub == 0 && slice == 0) {
    // lse of the group's heads: the threads whose chunk sits in column block 0, g == 0
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const int lc = tid + kThreads * k;
      if (lc < 16)
#pragma unroll
        for (int a = 0; a < 2; ++a)
          p.lse[orow + 16 * a + r16[k]] = wsum[k][a] > 0.f ? m[k][a] + __logf(wsum[k][a]) : kNegInf;
    }
  }
  __syncthreads();
  if (sub > 0) return;
  // row order: float4 e of the slice is head e / (4 CB), columns 16 CB slice + 4 (e % (4 CB)) .. +3
#pragma unroll
  for (int k = 0; k < 2 * kPerThread; ++k) {
    const int e = tid + kThreads * k;
    const int hl = e / (4 * CB), cc = e % (4 * CB);
    const int c = kRun * (hl >> 4) + 64 * (cc >> 2) + 16 * (cc & 3) + (hl & 15);
    float4* dst = (float4*)(p.out + (orow + hl) * kLatent + 16 * CB * slice) + cc;
    *dst = s_tile[lds_slot(c)];
  }
}

}  // namespace

template <int KC4, int KC8, int TS>
void launch_slices(const CombineParams& p, long long base, hipStream_t stream) {
  const long long want = 2048;
  if (base * 4 >= want) {
    // at most 512 threads a workgroup: 1024 would cap a thread at 128 VGPRs
    constexpr int TS2 = TS > 2 ? 2 : TS;
    combine_kernel<8, KC8, TS2><<<dim3((unsigned)(base * 4)), dim3(256 * TS2), 0, stream>>>(p);
  } else if (base * 8 >= want) {
    constexpr int TS2 = TS > 2 ? 2 : TS;
    combine_kernel<4, KC4, TS2><<<dim3((unsigned)(base * 8)), dim3(256 * TS2), 0, stream>>>(p);
  } else {
    combine_kernel<2, KC4, TS><<<dim3((unsigned)(base * 16)), dim3(128 * TS), 0, stream>>>(p);
  }
}

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
  // widest column slice that still gives about eight workgroups per compute
  // unit: the shares of short and long sequences then mix on every unit.
  // Partitions merged per memory round trip: 4, or, when sequences average
  // 16 partitions or more (a few long sequences), 16 (8 with two chunks a
  // thread) by each of four thread groups (two for the wider slices) sharing
  // a sequence's partitions.  Measured with rocprofv3: 17.2 -> 14.5 us on
  // 4 x 128k rows for the wider chunk, 13.0 -> 11.0 us for the groups (the
  // launch had 512 waves on the GPU); on 32 x 1k-4k and the paged mix the
  // wider chunk would cost 18% and 52% (fewer resident waves, merges of
  // partitions that are not there), two groups 17% and 39% (more merge work
  // in launches that already have 2048 workgroups).
  const long long base = (long long)p.batch * p.s_q * (kHeads / kGroupHeads);
  if ((long long)p.num_parts >= 16LL * p.batch) {
    launch_slices<16, 8, 4>(p, base, stream);
  } else {
    launch_slices<4, 4, 1>(p, base, stream);
  }
  return hipGetLastError();
}

}  // namespace mla
