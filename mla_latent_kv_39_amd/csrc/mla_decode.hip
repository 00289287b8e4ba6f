// Split-KV MLA decode kernel for gfx950 (bf16 latent cache).
//
// One workgroup (4 waves, one per SIMD) walks the 64-row units of one work
// partition.  Each unit (one cache page, 64 rows x 576 bf16 = 72 KB) is copied
// HBM -> LDS with direct-to-LDS loads into a two-slot ring, one unit ahead of
// the compute.  Every wave owns 32 query rows (32 heads of one query token):
//
//   scores  S^T[32 rows x 32 heads] = C[32 x 576] . Q^T[576 x 32]   MFMA 16x16x32 bf16
//   softmax online, per head, in fp32 (log2 domain), P rounded to bf16
//   output  O^T[512 x 32 heads]    += C^T[512 x 32] . P^T[32 x 32]  MFMA 16x16x32 bf16
//
// The score and output products read the same LDS tile: the cached latent is
// both the key and the value (DeepSeek-V3 architecture notes, deepseek.csdn.net,
// §2.1.2: k^C and v^C both expand the same c^KV; §2.1.3(B): W^UK sits in the
// query, W^UV after the call).  The output product needs the tile with rows
// along the reduction, which ds_read_b64_tr_b16 delivers from the row-major
// tile.  Q (32 heads x 576, 144 VGPRs) and O (32 heads x 512 fp32, 256
// registers) stay in registers for a whole sequence segment.
#include "mla_internal.h"
#include "mla_schedule.h"

namespace mla {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kChunks = kRow * 2 / 16;                    // 72 16-byte chunks per row
constexpr int kSlotBytes = kPage * kRowBytesBf16;         // 73728
constexpr int kSlots = 2;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.69314718055994530942f;

// Tile layout in LDS: chunk-column major.  16-byte chunk k (latent values
// 8k..8k+7) of the 64 rows of a unit occupies the 1 KB at k * 1024, row r at
// slot r ^ (8 * (k & 1)).  One wave instruction of the direct-to-LDS copy fills
// exactly one chunk column.  The score product reads 16 rows of one chunk
// (256 contiguous bytes); the transposing reads of the output product read
// 4 rows x 32 bytes from two neighbouring chunks, which the row XOR moves to
// different banks.
__device__ __forceinline__ int tile_offset(int row, int chunk) {
  return chunk * 1024 + ((row ^ (8 * (chunk & 1))) * 16);
}

__device__ __forceinline__ bf16x8 lds_read_b128(const lds_char* base, int off) {
  return *(const lds_bf16x8*)(base + off);
}

__device__ __forceinline__ i16x4 lds_read_tr(const lds_char* base, int off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + off));
}

__device__ __forceinline__ bf16x8 join(i16x4 lo, i16x4 hi) {
  typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8;
  i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Workgroup barrier for the tile ring.  __syncthreads() would also fence
// global memory and so wait for the direct-to-LDS copy still in flight; the
// ring only needs the LDS side ordered, which the explicit vmcnt waits before
// the barrier and the lgkmcnt wait here provide.  The asm statement is also a
// compiler barrier for memory accesses.
__device__ __forceinline__ void tile_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ float xor_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}

__device__ __forceinline__ float xor_sum(float v) {
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

// Copy one 64-row unit into an LDS slot: wave w fills chunk columns
// 18w .. 18w+17, lane L loading row L ^ (8 * (k & 1)) of column k.  Rows at or
// past `valid_rows` are fetched from row 0 of the same page instead, so stale
// page tails (which may hold any bits) never reach the tile.
__device__ __forceinline__ void load_unit(const char* page, int valid_rows, lds_char* slot, int wave, int lane) {
  const int r_even = lane, r_odd = lane ^ 8;
  const char* base_even = page + (r_even < valid_rows ? r_even : 0) * kRowBytesBf16;
  const char* base_odd = page + (r_odd < valid_rows ? r_odd : 0) * kRowBytesBf16;
  const int k0 = wave * (kChunks / 4);
#pragma unroll
  for (int i = 0; i < kChunks / 4; ++i) {
    const int k = k0 + i;  // k0 is even, so k & 1 == i & 1
    const char* src = ((i & 1) ? base_odd : base_even) + k * 16;
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(slot + k * 1024), 16, 0, 0);
  }
}

template <int SQ, int HB>
__global__ __launch_bounds__(256, 1) void decode_bf16_kernel(DecodeParams p) {
  static_assert(SQ * HB == 128, "four waves of 32 query rows");
  constexpr int NHB = kHeads / HB;
  constexpr float kHeadroom = 30.f;    // log2 units between the first max and the reference
  constexpr float kMaxExcess = 64.f;   // largest z - m_ref accepted before a restart
  __shared__ __attribute__((aligned(1024))) char smem[kSlots * kSlotBytes];
  __shared__ int s_scan[256];
  __shared__ int s_first[2];
  __shared__ int s_restart;
  lds_char* lds = (lds_char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;
  const int r16 = lane & 15;

  // Workgroup -> (partition, head block).  The NHB workgroups of one partition
  // are launched 8 apart, so they land on the same XCD and share its L2.
  int part, hblk;
  if (NHB == 1) {
    part = blockIdx.x;
    hblk = 0;
  } else if ((p.num_parts & 7) == 0) {
    const int xcd = blockIdx.x & 7, k = blockIdx.x >> 3;
    part = (k / NHB) * 8 + xcd;
    hblk = k % NHB;
  } else {
    part = blockIdx.x / NHB;
    hblk = blockIdx.x % NHB;
  }

  // ---- partition map: units of every sequence, prefix sums, this partition's range
  const int B = p.batch;
  const int per = (B + 255) >> 8;
  const int b_lo = min(B, tid * per), b_hi = min(B, b_lo + per);
  int cnt = 0;
  for (int b = b_lo; b < b_hi; ++b) cnt += units_of_len(p.seq_lens[b]);
  int total_units;
  const int excl = block_exclusive_scan_256(cnt, s_scan, &total_units);
  total_units = __builtin_amdgcn_readfirstlane(total_units);
  const int ua = part_start(part, total_units, p.num_parts);
  const int ub = part_start(part + 1, total_units, p.num_parts);
  if (ua >= ub) return;
  if (cnt > 0 && excl <= ua && ua < excl + cnt) {
    int b = b_lo, pre = excl;
    while (pre + units_of_len(p.seq_lens[b]) <= ua) {
      pre += units_of_len(p.seq_lens[b]);
      ++b;
    }
    s_first[0] = b;
    s_first[1] = pre;
  }
  if (tid == 0) s_restart = 0;
  __syncthreads();
  const int first_seq = __builtin_amdgcn_readfirstlane(s_first[0]);
  const int first_pre = __builtin_amdgcn_readfirstlane(s_first[1]);

  // ---- this wave's 32 query rows: token s_tok, heads head0 .. head0 + 31
  const int s_tok = (32 * wave) / HB;
  const int head0 = hblk * HB + (32 * wave) % HB;

  // lane-constant LDS offsets of the operand reads (see tile_offset)
  const int qk_off = tile_offset(r16, g);                        // + 4096 ks + 512 ss + 256 tb
  const int pv_off = tile_offset(4 * g + (r16 >> 2), (r16 & 3) >> 1) + (r16 & 1) * 8;  // + 2048 cb + 512 ss

  // loader cursor: runs one unit ahead of the compute
  int l_seq = first_seq, l_pre = first_pre, l_units = units_of_len(p.seq_lens[first_seq]);
  auto issue = [&](int u, int slot) {
    while (u >= l_pre + l_units) {
      l_pre += l_units;
      ++l_seq;
      l_units = units_of_len(p.seq_lens[l_seq]);
    }
    const int j = u - l_pre;
    const int valid = min(kPage, p.seq_lens[l_seq] - kPage * j);
    const char* page = p.rows;  // nothing visible: read page 0 row 0 (never used)
    if (valid > 0) {
      const long pg = p.block_table ? (long)p.block_table[(long)l_seq * p.max_blocks + j]
                                    : (long)l_seq * p.max_blocks + j;
      page = p.rows + pg * kSlotBytes;
    }
    load_unit(page, valid, lds + slot * kSlotBytes, wave, lane);
  };

  issue(ua, 0);
  int u = ua;
  int c_seq = first_seq, c_pre = first_pre;
  while (u < ub) {
    // ---- one segment: this partition's units of sequence c_seq
    const int c_len = p.seq_lens[c_seq];
    const int c_units = units_of_len(c_len);
    const int seg_end = min(ub, c_pre + c_units);
    const int nvis = c_len - SQ + s_tok + 1;  // rows this wave's query token sees

    bf16x8 qf[18][2];
    f32x4 O[32][2];
    float m_ref[2], l_run[2];
    {
      const size_t qrow = (size_t)(c_seq * SQ + s_tok) * kHeads + head0;
      const __bf16* qa = p.q_abs + qrow * kLatent;
      const __bf16* qr = p.q_rope + qrow * kRope;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int ks = 0; ks < 16; ++ks)
          qf[ks][h] = *(const bf16x8*)(qa + (16 * h + r16) * kLatent + 32 * ks + 8 * g);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          qf[16 + ks][h] = *(const bf16x8*)(qr + (16 * h + r16) * kRope + 32 * ks + 8 * g);
        m_ref[h] = kNegInf;
        l_run[h] = 0.f;
#pragma unroll
        for (int cb = 0; cb < 32; ++cb) O[cb][h] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }

    for (; u < seg_end; ++u) {
      const int slot = (u - ua) & 1;
      if (u + 1 < ub) {
        issue(u + 1, slot ^ 1);
        __builtin_amdgcn_s_waitcnt(0x4F72);  // vmcnt(18): all but the 18 loads just issued
      } else {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      }
      tile_barrier();

      const lds_char* tile = lds + slot * kSlotBytes;
      const int row0 = kPage * (u - c_pre);
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
        if (nvis > row0 + 32 * ss) {
          // S^T = C Q^T for 32 rows x 32 heads
          f32x4 acc[2][2];
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int h = 0; h < 2; ++h) acc[tb][h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 18; ++ks) {
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
              const bf16x8 a = lds_read_b128(tile, qk_off + 4096 * ks + 512 * ss + 256 * tb);
              acc[tb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[ks][0], acc[tb][0], 0, 0, 0);
              acc[tb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[ks][1], acc[tb][1], 0, 0, 0);
            }
          }
          // Softmax in the log2 domain against a reference m_ref that is fixed for
          // the segment: at its first visible rows m_ref = their max + kHeadroom, and
          // P = 2^(z - m_ref) from then on.  O therefore never needs rescaling.  If a
          // later max passes m_ref + kMaxExcess (P could approach the fp32 range),
          // m_ref is raised and the whole workgroup restarts the segment.
          float z[2][2][4];
          bool over = false;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            float mx = kNegInf;
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int pos = row0 + 32 * ss + 16 * tb + 4 * g + i;
                z[h][tb][i] = pos < nvis ? acc[tb][h][i] * p.scale_log2 : kNegInf;
                mx = fmaxf(mx, z[h][tb][i]);
              }
            mx = xor_max(mx);
            if (m_ref[h] == kNegInf && mx != kNegInf) m_ref[h] = mx + kHeadroom;
            if (mx > m_ref[h] + kMaxExcess) {
              m_ref[h] = mx + kHeadroom;
              over = true;
            }
          }
          if (__builtin_expect(__builtin_amdgcn_ballot_w64(over) != 0, 0)) s_restart = 1;
          bf16x8 pb[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const float ref = m_ref[h] == kNegInf ? 0.f : m_ref[h];  // all rows masked so far
            float sum = 0.f;
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                z[h][tb][i] = __builtin_amdgcn_exp2f(z[h][tb][i] - ref);
                sum += z[h][tb][i];
              }
            l_run[h] += sum;
            pb[h] = bf16x8{(__bf16)z[h][0][0], (__bf16)z[h][0][1], (__bf16)z[h][0][2], (__bf16)z[h][0][3],
                           (__bf16)z[h][1][0], (__bf16)z[h][1][1], (__bf16)z[h][1][2], (__bf16)z[h][1][3]};
          }
          // O += P C: B operand = 32 rows x 16 latent columns, transposed out of the tile
#pragma unroll
          for (int cb = 0; cb < 32; ++cb) {
            const int off = pv_off + 2048 * cb + 512 * ss;
            const bf16x8 c = join(lds_read_tr(tile, off), lds_read_tr(tile, off + 256));
            O[cb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pb[0], c, O[cb][0], 0, 0, 0);
            O[cb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pb[1], c, O[cb][1], 0, 0, 0);
          }
        }
      }
      tile_barrier();
      if (__builtin_expect(s_restart != 0, 0)) {
        // some head's max outran its reference: drain the copy in flight and redo
        // the segment from its first unit with the raised references
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        tile_barrier();
        if (tid == 0) s_restart = 0;
        u = max(ua, c_pre) - 1;  // the loop increment brings it to the segment start
        l_seq = c_seq;
        l_pre = c_pre;
        l_units = c_units;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          l_run[h] = 0.f;
#pragma unroll
          for (int cb = 0; cb < 32; ++cb) O[cb][h] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        issue(u + 1, (u + 1 - ua) & 1);
        tile_barrier();
      }
    }

    // ---- end of segment: normalise and store (final result or a partial).
    // O layout: lane holds heads 4g+i (i < 4) of head block h, column 16 cb + r16;
    // the softmax statistics of head r16 live in every lane with that r16.
    const bool whole = c_pre >= ua && c_pre + c_units <= ub;
    const int pslot = c_pre <= ua ? 0 : 1;
    const size_t row_base = whole ? (size_t)(c_seq * SQ + s_tok) * kHeads
                                  : ((size_t)(part * 2 + pslot) * SQ + s_tok) * kHeads;
    float* out_base = whole ? p.out : p.part_out;
    float* lse_base = whole ? p.lse : p.part_lse;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float lt = xor_sum(l_run[h]);
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      if (g == 0) lse_base[row_base + head0 + 16 * h + r16] = lt > 0.f ? (m_ref[h] + __log2f(lt)) * kLn2 : kNegInf;
      float inv_i[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) inv_i[i] = __shfl(inv, 4 * g + i);
#pragma unroll
      for (int cb = 0; cb < 32; ++cb) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          out_base[(row_base + head0 + 16 * h + 4 * g + i) * kLatent + 16 * cb + r16] = O[cb][h][i] * inv_i[i];
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    c_pre += c_units;
    ++c_seq;
  }
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeParams& p, int s_q, hipStream_t stream) {
  if (s_q == 1) {
    decode_bf16_kernel<1, 128><<<dim3(p.num_parts), dim3(256), 0, stream>>>(p);
  } else {
    decode_bf16_kernel<2, 64><<<dim3(p.num_parts * 2), dim3(256), 0, stream>>>(p);
  }
  return hipGetLastError();
}

}  // namespace mla

namespace mla {
// The e4m3 cache path is not built yet.
hipError_t launch_decode_fp8(const DecodeParams&, int, hipStream_t) { return hipErrorNotSupported; }
}  // namespace mla
