// The steps around the decode in one MLA attention layer (DeepSeek-V3
// architecture notes, deepseek.csdn.net, §2.1.2 and §2.1.3(B), (D)):
//
//   absorbed query   q_absorbed_h = W^UK_h^T q^C_h         (per head, 128 -> 512)
//   query RoPE       q_rope = RoPE(q^R, position)
//   output values    o_h = W^UV_h out_latent_h              (per head, 512 -> 128)
//   KV projection    [c^KV ; k] = [W^DKV ; W^KR] h          (d -> 512 + 64)
//   cache append     row = [c^KV ; RoPE(k, position)] into its page slot,
//                    bf16, or e4m3 with one fp32 scale per 128 values
//                    (DeepSeek-V3 详解, yudonglee.me, §4.2)
//
// The three projections are C[M x N] = A[M x K] W[N x K]^T on bf16 MFMA
// (v_mfma_f32_16x16x32_bf16) with fp32 accumulation, batched over heads for
// the two absorptions.  M is the number of tokens of a decode step (a few
// hundred): every weight byte serves every token of its tile, so the kernels
// are bound by the weight and activation bytes.  The two absorptions stage
// their operands through LDS (each line crosses a compute unit's L1 once,
// with loads always in flight); the projection, whose K of 7168 leaves few
// output tiles, splits K over the waves of a workgroup and loads its operands
// straight into MFMA registers.  Outputs come out of the MFMAs four
// consecutive columns per lane; the absorptions and the split projection
// pass them through LDS so that whole row segments are stored.
#include <hip/hip_bf16.h>

#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// Raw operand fragments: 8 consecutive K values of one row, as loaded (16
// bytes of bf16, or 32 bytes of fp32 rounded to bf16 only when used, so that
// the rounding never waits on a load that the pipeline wants in flight).
template <typename T>
struct Raw;
template <>
struct Raw<__bf16> {
  uint4 u;
  __device__ __forceinline__ void load(const __bf16* p, bool ok) {
    u = ok ? *reinterpret_cast<const uint4*>(p) : make_uint4(0, 0, 0, 0);
  }
  __device__ __forceinline__ bf16x8 frag() const { return __builtin_bit_cast(bf16x8, u); }
};
template <>
struct Raw<float> {
  float4 lo, hi;
  __device__ __forceinline__ void load(const float* p, bool ok) {
    lo = hi = make_float4(0.f, 0.f, 0.f, 0.f);
    if (ok) {
      lo = reinterpret_cast<const float4*>(p)[0];
      hi = reinterpret_cast<const float4*>(p)[1];
    }
  }
  __device__ __forceinline__ bf16x8 frag() const {   // round to nearest even
    bf16x8 r;
    r[0] = (__bf16)lo.x;
    r[1] = (__bf16)lo.y;
    r[2] = (__bf16)lo.z;
    r[3] = (__bf16)lo.w;
    r[4] = (__bf16)hi.x;
    r[5] = (__bf16)hi.y;
    r[6] = (__bf16)hi.z;
    r[7] = (__bf16)hi.w;
    return r;
  }
};

// four consecutive outputs: one 16-byte (fp32) or 8-byte (bf16) store
__device__ __forceinline__ void store4(float* p, const floatx4& v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store4(__bf16* p, const floatx4& v) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 h;
  h[0] = (__bf16)v[0];
  h[1] = (__bf16)v[1];
  h[2] = (__bf16)v[2];
  h[3] = (__bf16)v[3];
  *reinterpret_cast<bf16x4*>(p) = h;
}

// C (m, n) = sum_k A (m, k) W (n, k), batch z:
//   A (m, k) at a + z a_batch + m a_row + k,  W (n, k) at w + z w_batch + n k_len + k,
//   C (m, n) at c + z c_batch + m c_row + n.
// The MFMA takes W as its first operand and A as its second, so a 16 x 16
// block comes out transposed: lane (r16, g) holds C (m = r16, n = 4g .. 4g+3),
// four consecutive outputs of one row, stored straight from the accumulators.
// The NW = KW waves own the same (16 WM) x (16 WN) outputs, each over 1/KW
// of K (for long K and few outputs); their partial tiles are summed in LDS in
// a fixed order.  K is walked in stages of U
// K-steps (32 U values) with two register buffers: the loads of stage s + 1
// are issued before the MFMAs of stage s, so a wave always has a stage of
// loads in flight.  Requires k_len % (32 KW) == 0 and n_len a multiple of the
// tile width; rows m >= m_len are neither read nor written.
template <typename TA, typename TC, int WM, int WN, int KW, int NW, int U>
__global__ __launch_bounds__(64 * NW) void gemm_nt_kernel(GemmParams g) {
  static_assert(KW == NW && KW > 1, "all waves over K");
  constexpr int TM = 16 * WM;
  constexpr int TN = 16 * WN;
  constexpr int PITCH = TN + 4;                  // floats per LDS row (K split only)
  __shared__ float s_tile[NW * TM * PITCH];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, kg = lane >> 4;
  const int wm0 = 0, wn0 = 0;      // every wave covers the whole tile
  const int m0 = blockIdx.y * TM + wm0;
  const int n0 = blockIdx.x * TN + wn0;
  const int kq = g.k_len / KW;
  const int kbeg = wave * kq;
  const int64_t z = blockIdx.z;
  const TA* A = static_cast<const TA*>(g.a) + z * g.a_batch;
  const __bf16* W = g.w + z * g.w_batch;
  const TA* arow[WM];
  bool aok[WM];
#pragma unroll
  for (int i = 0; i < WM; ++i) {
    const int m = m0 + 16 * i + r16;
    aok[i] = m < g.m_len;
    arow[i] = A + (int64_t)(aok[i] ? m : 0) * g.a_row + kbeg + 8 * kg;
  }
  const __bf16* wrow[WN];
#pragma unroll
  for (int j = 0; j < WN; ++j) wrow[j] = W + (int64_t)(n0 + 16 * j + r16) * g.k_len + kbeg + 8 * kg;
  floatx4 acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  Raw<TA> ra[2][U][WM];
  Raw<__bf16> rw[2][U][WN];
  auto load = [&](int buf, int k) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int j = 0; j < WN; ++j) rw[buf][u][j].load(wrow[j] + k + 32 * u, true);
#pragma unroll
      for (int i = 0; i < WM; ++i) ra[buf][u][i].load(arow[i] + k + 32 * u, aok[i]);
    }
  };
  auto compute = [&](int buf) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        const bf16x8 x = ra[buf][u][i].frag();
#pragma unroll
        for (int j = 0; j < WN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rw[buf][u][j].frag(), x, acc[i][j], 0, 0, 0);
      }
  };
  const int nst = kq / (32 * U);
  int st = 0;
  if (nst > 0) load(0, 0);
  for (; st + 2 <= nst; st += 2) {
    load(1, (st + 1) * 32 * U);
    compute(0);
    if (st + 2 < nst) load(0, (st + 2) * 32 * U);
    compute(1);
  }
  if (st < nst) compute(0);
  for (int k = nst * 32 * U; k < kq; k += 32) {   // K-steps past the last whole stage
#pragma unroll
    for (int j = 0; j < WN; ++j) rw[0][0][j].load(wrow[j] + k, true);
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      ra[0][0][i].load(arow[i] + k, aok[i]);
      const bf16x8 x = ra[0][0][i].frag();
#pragma unroll
      for (int j = 0; j < WN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rw[0][0][j].frag(), x, acc[i][j], 0, 0, 0);
    }
  }

  TC* C = static_cast<TC*>(g.c) + z * g.c_batch;
  // K split: the NW partial tiles summed in LDS, then written row by row
  float* mine = s_tile + wave * TM * PITCH;
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
      *reinterpret_cast<float4*>(mine + (16 * i + r16) * PITCH + 16 * j + 4 * kg) =
          make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
  __syncthreads();
  const int mt = blockIdx.y * TM, nt = blockIdx.x * TN;
  for (int e = threadIdx.x; e < TM * (TN / 4); e += 64 * NW) {
    const int r = e / (TN / 4), c4 = (e % (TN / 4)) * 4;
    if (mt + r >= g.m_len) continue;
    floatx4 v = *reinterpret_cast<const floatx4*>(s_tile + r * PITCH + c4);
#pragma unroll
    for (int w = 1; w < NW; ++w) v += *reinterpret_cast<const floatx4*>(s_tile + (w * TM + r) * PITCH + c4);
    store4(C + (int64_t)(mt + r) * g.c_row + nt + c4, v);
  }
}

// q_rope of query token t = b S_q + s by one workgroup of 256 threads,
// position seq_len[b] - S_q + s, in three steps: each thread loads its 16
// pairs (8-byte loads of two pairs), threads 0..31 compute the 32 angles'
// cosines and sines once for the token (fp64) into LDS, and after a barrier
// every thread rotates its pairs.
struct QueryRopeToken {
  static constexpr int kPer = kHeads * kRope / 4 / 256;   // groups of four values per thread
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 x[kPer];
  int64_t base;
  int pos;
  __device__ __forceinline__ void load(const RopeParams& p, int t) {
    base = (int64_t)t * kHeads * kRope;
    pos = p.seq_lens[t / p.s_q] - p.s_q + t % p.s_q;
#pragma unroll
    for (int k = 0; k < kPer; ++k) x[k] = *reinterpret_cast<const bf16x4*>(p.src + base + 4 * (threadIdx.x + 256 * k));
  }
  __device__ __forceinline__ void angles(const RopeParams& p, float (*s_cs)[kRope / 2]) const {
    if (threadIdx.x < kRope / 2) {
      const double theta = pow(p.base, -2.0 * (double)threadIdx.x / (double)kRope);
      double sn, cs;
      sincos((double)pos * theta, &sn, &cs);
      s_cs[0][threadIdx.x] = (float)cs;
      s_cs[1][threadIdx.x] = (float)sn;
    }
  }
  __device__ __forceinline__ void rotate_store(const RopeParams& p, const float (*s_cs)[kRope / 2]) const {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int e = threadIdx.x + 256 * k;
      const int i = (e % (kRope / 4)) * 2;                         // first pair of the four values
      bf16x4 y;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const float c = s_cs[0][i + q], sn = s_cs[1][i + q];
        const float x0 = (float)x[k][2 * q], x1 = (float)x[k][2 * q + 1];
        y[2 * q] = (__bf16)fmaf(x0, c, -x1 * sn);
        y[2 * q + 1] = (__bf16)fmaf(x0, sn, x1 * c);
      }
      *reinterpret_cast<bf16x4*>(p.dst + base + 4 * e) = y;
    }
  }
};

// Absorbed query q_absorbed_h = W^UK_h^T q^C_h (K = 128, N = 512 per head),
// and q_rope = RoPE(q^R, position) in the same launch: one workgroup per
// (head, tile of 128 tokens), every tile of a head on one XCD (blockIdx.x is
// the head: workgroups are dealt to the 8 XCDs by linear id), so the head's
// weight is fetched from HBM once.  The token tile stays in LDS; the weight
// goes through in four chunks of 128 output columns, two LDS buffers, each
// thread keeping two chunks of loads in registers so that they are in
// flight while a chunk's MFMAs run and its outputs are stored (loading the
// weight and the tiles first and storing after them measured 20 us for 256
// tokens).  LDS rows are 256 bytes (16 chunks of 16 bytes); chunk c of row r
// sits at chunk c ^ (r & 15), so the 16 rows of an operand fragment read
// (one chunk each) hit 16 different chunk positions of the bank row.
// Workgroup i also rotates the q^R of tokens i, i + grid, ... (all heads;
// each token's angles are evaluated once), token i's while the first loads
// are in flight.  (Rotating each head's pairs in that head's workgroups
// instead evaluates every angle 128 times: 24.6 us against 22.4 us for a
// GEMM and a separate RoPE kernel.)
constexpr int kAqTileM = 128;
constexpr int kAqChunkN = 128;                // output columns per weight chunk
constexpr int kAqN = 512;                     // d_c
constexpr int kAqK = 128;                     // d_h: the chunks of a row
constexpr int kAqChunks = kAqK / 8;           // 16-byte chunks per row
constexpr int kAqNChunks = kAqN / kAqChunkN;
constexpr int kAqPer = kAqTileM * kAqChunks / 256;   // 16-byte chunks per thread of a tile (8)

__device__ __forceinline__ int aq_slot(int r, int c) { return r * kAqChunks + (c ^ (r & 15)); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
struct AqRegs {
  u32x4 v[kAqPer];
};
template <int N>
struct IntC {
  static constexpr int value = N;
};

__global__ __launch_bounds__(256) void absorb_query_kernel(GemmParams g, RopeParams rp) {
  __shared__ u32x4 s_a[kAqTileM * kAqChunks];            // 32 KB
  __shared__ u32x4 s_w[2][kAqChunkN * kAqChunks];        // 2 x 32 KB
  __shared__ u32x4 s_c[4][64 * 8];                         // 4 x 8 KB: each wave's outputs of a chunk
  __shared__ float s_cs[2][kRope / 2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, kg = lane >> 4;
  const int head = blockIdx.x, m0 = blockIdx.y * kAqTileM;
  const int id = blockIdx.x + gridDim.x * blockIdx.y;
  const __bf16* A = static_cast<const __bf16*>(g.a) + (int64_t)head * g.a_batch + (int64_t)m0 * g.a_row;
  const __bf16* W = g.w + (int64_t)head * g.w_batch;
  __bf16* C = static_cast<__bf16*>(g.c) + (int64_t)head * g.c_batch;
  const int mrows = g.m_len - m0;               // >= 1; token rows past it are read as its last one
  // thread t moves chunks e = t + 256 i: row e / 16, chunk e % 16 (16 threads
  // per 256-byte row: a wave's load covers four whole rows)
  auto load_a = [&](AqRegs& r) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kAqPer; ++i) {
      const int e = tid + 256 * i, row = e / kAqChunks;
      const int rr = row < mrows ? row : mrows - 1;
      r.v[i] = *reinterpret_cast<const u32x4*>(A + (int64_t)rr * g.a_row + 8 * (e % kAqChunks));
    }
  };
  auto load_w = [&](AqRegs& r, int chunk) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kAqPer; ++i) {
      const int e = tid + 256 * i;
      r.v[i] = *reinterpret_cast<const u32x4*>(W + (int64_t)(chunk * kAqChunkN + e / kAqChunks) * kAqK +
                                               8 * (e % kAqChunks));
    }
  };
  auto put = [&](const AqRegs& r, u32x4* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kAqPer; ++i) {
      const int e = tid + 256 * i;
      dst[aq_slot(e / kAqChunks, e % kAqChunks)] = r.v[i];
    }
  };
  QueryRopeToken rt;
  const bool rope0 = id < rp.tokens;          // uniform over the workgroup
  if (rope0) rt.load(rp, id);
  AqRegs ra, rw0, rw1;
  load_a(ra);
  load_w(rw0, 0);
  load_w(rw1, 1);
  if (rope0) rt.angles(rp, s_cs);
  put(ra, s_a);
  put(rw0, s_w[0]);
  load_w(rw0, 2);
  __syncthreads();
  if (rope0) rt.rotate_store(rp, s_cs);

  // wave (wm, wn) owns tokens 64 wm .. +63 and columns 64 wn .. +63 of a chunk
  const int wm = wave & 1, wn = wave >> 1;
  auto chunk = [&](auto cc) __attribute__((always_inline)) {
    constexpr int c = decltype(cc)::value;
    const u32x4* sw = s_w[c & 1];
    floatx4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kAqK / 32; ++u) {
      bf16x8 x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = __builtin_bit_cast(bf16x8, s_a[aq_slot(64 * wm + 16 * i + r16, 4 * u + kg)]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8 wf = __builtin_bit_cast(bf16x8, sw[aq_slot(64 * wn + 16 * j + r16, 4 * u + kg)]);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, x[i], acc[i][j], 0, 0, 0);
      }
    }
    // chunk c + 1 into the buffer whose last readers passed the previous
    // barrier, then its registers take chunk c + 3
    if constexpr (c + 1 < kAqNChunks && ((c + 1) & 1)) {
      put(rw1, s_w[1]);
      if constexpr (c + 3 < kAqNChunks) load_w(rw1, c + 3);
    } else if constexpr (c + 1 < kAqNChunks) {
      put(rw0, s_w[0]);
      if constexpr (c + 3 < kAqNChunks) load_w(rw0, c + 3);
    }
    // outputs through this wave's own LDS area, so that they leave as whole
    // 128-byte row segments (16 bytes a lane) instead of 8 bytes a lane, 16
    // rows x 32 bytes a store.  Lane (r16, kg) of block (i, j) holds token
    // 16 i + r16, columns 16 j + 4 kg .. +3 of the wave's 64 x 64 block; a row
    // is 8 chunks of 16 bytes, chunk q at q ^ ((r >> 1) & 7).
    u32x4* sc = s_c[wave];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * i + r16, q = 2 * j + (kg >> 1);
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 h;
        h[0] = (__bf16)acc[i][j][0];
        h[1] = (__bf16)acc[i][j][1];
        h[2] = (__bf16)acc[i][j][2];
        h[3] = (__bf16)acc[i][j][3];
        *reinterpret_cast<bf16x4*>(reinterpret_cast<char*>(sc + r * 8 + (q ^ ((r >> 1) & 7))) + 8 * (kg & 1)) = h;
      }
    // the reads below take other lanes' writes: a wave's LDS instructions
    // complete in order, and the compiler must not move the reads above them
    asm volatile("" ::: "memory");
    // lane L stores chunk L % 8 of rows L / 8 + 8 t: columns 128 c + 64 wn + 8 (L % 8) .. +7
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int r = lane / 8 + 8 * t, q = lane % 8;
      const u32x4 v = sc[r * 8 + (q ^ ((r >> 1) & 7))];
      const int m = m0 + 64 * wm + r;
      if (m < g.m_len)
        *reinterpret_cast<u32x4*>(C + (int64_t)m * g.c_row + kAqChunkN * c + 64 * wn + 8 * q) = v;
    }
    __syncthreads();
  };
  chunk(IntC<0>{});
  chunk(IntC<1>{});
  chunk(IntC<2>{});
  chunk(IntC<3>{});
  static_assert(kAqNChunks == 4, "one call per chunk above");
  // more tokens than workgroups: the rest of this workgroup's share (s_cs is
  // free: every thread has passed the barrier after its last reader)
  const int grid = (int)(gridDim.x * gridDim.y);
  for (int t = id + grid; t < rp.tokens; t += grid) {
    rt.load(rp, t);
    rt.angles(rp, s_cs);
    __syncthreads();
    rt.rotate_store(rp, s_cs);
    __syncthreads();
  }
}

// Output values o_h = W^UV_h out_latent_h (K = 512 fp32 values rounded to
// bf16 when used, N = 128 per head, fp32 out): one workgroup per (head, tile
// of 128 tokens), every tile of a head on one XCD (blockIdx.x is the head:
// workgroups are dealt to the 8 XCDs by linear id), so its weight is fetched
// from HBM once.  K runs in 8 stages of 64 through two LDS buffers; each
// thread keeps two stages of loads in registers, so two are always in flight
// while a stage's MFMAs run (direct-to-LDS loads would need the compiler to
// wait for every load in flight before any LDS read: with them, one stage at
// a time, 25.5 us for 256 tokens).  LDS rows: the tokens' 64 fp32 values as
// 16 chunks of 16 bytes, chunk c at c ^ (r & 15); the weight's 64 bf16
// values as 8 chunks, chunk c at c ^ ((r >> 1) & 7) (two 128-byte rows per
// bank row): the 16 rows of a fragment read fall on 16 different bank
// positions.
constexpr int kAoTileM = 128;
constexpr int kAoN = 128;                     // d_h
constexpr int kAoK = 512;                     // d_c
constexpr int kAoStage = 64;                  // K values per stage
constexpr int kAoStages = kAoK / kAoStage;
constexpr int kAoAChunks = kAoStage / 4;      // fp32 chunks per token row of a stage (16)
constexpr int kAoWChunks = kAoStage / 8;      // bf16 chunks per weight row of a stage (8)
constexpr int kAoAPer = kAoTileM * kAoAChunks / 256;   // chunks per thread and stage: 8 of tokens,
constexpr int kAoWPer = kAoN * kAoWChunks / 256;       // 4 of weight

__device__ __forceinline__ int ao_wslot(int r, int c) { return r * kAoWChunks + (c ^ ((r >> 1) & 7)); }

// staging registers of one stage (clang vectors: HIP's uint4 is a class with
// union storage, which kept arrays of it out of registers)
struct AoStage {
  u32x4 a[kAoAPer], w[kAoWPer];
};

__global__ __launch_bounds__(256) void absorb_output_kernel(GemmParams g) {
  __shared__ u32x4 s_a[2][kAoTileM * kAoAChunks];      // 2 x 32 KB
  __shared__ u32x4 s_w[2][kAoN * kAoWChunks];          // 2 x 16 KB
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, kg = lane >> 4;
  const int head = blockIdx.x, m0 = blockIdx.y * kAoTileM;
  const float* A = static_cast<const float*>(g.a) + (int64_t)head * g.a_batch + (int64_t)m0 * g.a_row;
  const __bf16* W = g.w + (int64_t)head * g.w_batch;
  float* C = static_cast<float*>(g.c) + (int64_t)head * g.c_batch;
  const int mrows = g.m_len - m0;               // >= 1; token rows past it are read as its last one
  // thread t moves chunks e = t + 256 i: token row e / 16, chunk e % 16 (16
  // threads per 256-byte row); weight row e / 8, chunk e % 8
  auto load = [&](AoStage& r, int st) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kAoAPer; ++i) {
      const int e = tid + 256 * i, row = e / kAoAChunks;
      const int rr = row < mrows ? row : mrows - 1;
      r.a[i] = *reinterpret_cast<const u32x4*>(A + (int64_t)rr * g.a_row + st * kAoStage + 4 * (e % kAoAChunks));
    }
#pragma unroll
    for (int i = 0; i < kAoWPer; ++i) {
      const int e = tid + 256 * i;
      r.w[i] = *reinterpret_cast<const u32x4*>(W + (int64_t)(e / kAoWChunks) * kAoK + st * kAoStage +
                                               8 * (e % kAoWChunks));
    }
  };
  auto put = [&](const AoStage& r, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kAoAPer; ++i) {
      const int e = tid + 256 * i, row = e / kAoAChunks;
      s_a[buf][row * kAoAChunks + ((e % kAoAChunks) ^ (row & 15))] = r.a[i];
    }
#pragma unroll
    for (int i = 0; i < kAoWPer; ++i) {
      const int e = tid + 256 * i;
      s_w[buf][ao_wslot(e / kAoWChunks, e % kAoWChunks)] = r.w[i];
    }
  };
  // wave (wm, wn) owns tokens 64 wm .. +63 and columns 64 wn .. +63
  const int wm = wave & 1, wn = wave >> 1;
  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  // register set st % 2 holds stage st from its load until its LDS write
  // (two named sets and a compile-time stage index keep them in registers)
  AoStage rs0, rs1;
  load(rs0, 0);
  load(rs1, 1);
  put(rs0, 0);
  load(rs0, 2);
  __syncthreads();
  auto stage = [&](auto stc) __attribute__((always_inline)) {
    constexpr int st = decltype(stc)::value;
    const u32x4* sa = s_a[st & 1];
    const u32x4* sw = s_w[st & 1];
#pragma unroll
    for (int u = 0; u < kAoStage / 32; ++u) {
      bf16x8 x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 64 * wm + 16 * i + r16;
        Raw<float> raw;
        raw.lo = __builtin_bit_cast(float4, sa[r * kAoAChunks + ((8 * u + 2 * kg) ^ (r & 15))]);
        raw.hi = __builtin_bit_cast(float4, sa[r * kAoAChunks + ((8 * u + 2 * kg + 1) ^ (r & 15))]);
        x[i] = raw.frag();
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8 wf = __builtin_bit_cast(bf16x8, sw[ao_wslot(64 * wn + 16 * j + r16, 4 * u + kg)]);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, x[i], acc[i][j], 0, 0, 0);
      }
    }
    // stage st + 1 into the buffer whose last readers passed the previous
    // barrier, then its registers take stage st + 3
    if constexpr (st + 1 < kAoStages && ((st + 1) & 1)) {
      put(rs1, 1);
      if constexpr (st + 3 < kAoStages) load(rs1, st + 3);
    } else if constexpr (st + 1 < kAoStages) {
      put(rs0, 0);
      if constexpr (st + 3 < kAoStages) load(rs0, st + 3);
    }
    __syncthreads();
  };
  stage(IntC<0>{});
  stage(IntC<1>{});
  stage(IntC<2>{});
  stage(IntC<3>{});
  stage(IntC<4>{});
  stage(IntC<5>{});
  stage(IntC<6>{});
  stage(IntC<7>{});
  static_assert(kAoStages == 8, "one call per stage above");
  // outputs through LDS (the token buffers are free after the last barrier:
  // waves 2 w' and 2 w' + 1 take halves of buffer w'), so that they leave as
  // whole 256-byte row segments rather than 64 bytes of 16 rows a store.
  // Lane (r16, kg) of block (i, j) holds token 16 i + r16, columns 16 j +
  // 4 kg .. +3 of the wave's 64 x 64 block; a row is 16 chunks of 16 bytes,
  // chunk q at q ^ (r & 15).
  u32x4* sc = s_a[wave >> 1] + (wave & 1) * (64 * 16);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 16 * i + r16, q = 4 * j + kg;
      sc[r * 16 + (q ^ (r & 15))] = __builtin_bit_cast(u32x4, acc[i][j]);
    }
  // the reads below take other lanes' writes: a wave's LDS instructions
  // complete in order, and the compiler must not move the reads above them
  asm volatile("" ::: "memory");
  // lane L stores chunk L % 16 of rows L / 16 + 4 t: columns 64 wn + 4 (L % 16) .. +3
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const int r = lane / 16 + 4 * t, q = lane % 16;
    const u32x4 v = sc[r * 16 + (q ^ (r & 15))];
    const int m = m0 + 64 * wm + r;
    if (m < g.m_len) *reinterpret_cast<u32x4*>(C + (int64_t)m * g.c_row + 64 * wn + 4 * q) = v;
  }
}

// KV projection with K cut over workgroups (mla_kv_project_split): slice s of
// S takes K values [s K / S, (s + 1) K / S) of one tile of 128 tokens x 64
// output features and writes its fp32 partial sums to the caller's
// workspace [S, T, 576]; kv_reduce_kernel then adds the S partials of each
// output in slice order (the result does not depend on the order workgroups
// run in).  For a decode step's few hundred tokens this spreads the 7168-deep
// contraction over the whole GPU: each workgroup reads 192 KB of operands
// instead of the 0.9 MB a 32 x 32 tile over all of K takes.  K runs in
// stages of 64 through two LDS buffers, two stages of loads in registers
// (as in the output absorption); rows of both operands are 128 bytes per
// stage, 8 chunks, chunk c at c ^ ((r >> 1) & 7).
constexpr int kKvTileM = 128;
constexpr int kKvTileN = 64;
constexpr int kKvStage = 64;
constexpr int kKvChunks = kKvStage / 8;                    // 8 chunks of 16 bytes per row
constexpr int kKvAPer = kKvTileM * kKvChunks / 256;         // 4 chunks per thread and stage
constexpr int kKvWPer = kKvTileN * kKvChunks / 256;         // 2

struct KvStage {
  u32x4 a[kKvAPer], w[kKvWPer];
};

__global__ __launch_bounds__(256) void kv_partial_kernel(GemmParams g, float* ws, int slices) {
  __shared__ u32x4 s_a[2][kKvTileM * kKvChunks];   // 2 x 16 KB
  __shared__ u32x4 s_w[2][kKvTileN * kKvChunks];   // 2 x 8 KB
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, kg = lane >> 4;
  const int m0 = blockIdx.x * kKvTileM, n0 = blockIdx.y * kKvTileN, slice = blockIdx.z;
  const int klen = g.k_len / slices, k0 = slice * klen;
  const int nst = klen / kKvStage;                 // even: klen is a multiple of 128
  const __bf16* A = static_cast<const __bf16*>(g.a) + (int64_t)m0 * g.a_row + k0;
  const __bf16* W = g.w + (int64_t)n0 * g.k_len + k0;
  const int mrows = g.m_len - m0;                  // >= 1; token rows past it are read as its last one
  // thread t moves chunks e = t + 256 i: row e / 8, chunk e % 8 (8 threads per 128-byte row)
  auto load = [&](KvStage& r, int st) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kKvAPer; ++i) {
      const int e = tid + 256 * i, row = e / kKvChunks;
      const int rr = row < mrows ? row : mrows - 1;
      r.a[i] = *reinterpret_cast<const u32x4*>(A + (int64_t)rr * g.a_row + st * kKvStage + 8 * (e % kKvChunks));
    }
#pragma unroll
    for (int i = 0; i < kKvWPer; ++i) {
      const int e = tid + 256 * i;
      r.w[i] = *reinterpret_cast<const u32x4*>(W + (int64_t)(e / kKvChunks) * g.k_len + st * kKvStage +
                                               8 * (e % kKvChunks));
    }
  };
  auto put = [&](const KvStage& r, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kKvAPer; ++i) {
      const int e = tid + 256 * i;
      s_a[buf][ao_wslot(e / kKvChunks, e % kKvChunks)] = r.a[i];
    }
#pragma unroll
    for (int i = 0; i < kKvWPer; ++i) {
      const int e = tid + 256 * i;
      s_w[buf][ao_wslot(e / kKvChunks, e % kKvChunks)] = r.w[i];
    }
  };
  // wave (wm, wn) owns tokens 64 wm .. +63 and features 32 wn .. +31
  const int wm = wave & 1, wn = wave >> 1;
  floatx4 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kKvStage / 32; ++u) {
      bf16x8 x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = __builtin_bit_cast(bf16x8, s_a[buf][ao_wslot(64 * wm + 16 * i + r16, 4 * u + kg)]);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bf16x8 wf = __builtin_bit_cast(bf16x8, s_w[buf][ao_wslot(32 * wn + 16 * j + r16, 4 * u + kg)]);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, x[i], acc[i][j], 0, 0, 0);
      }
    }
  };
  // register set st % 2 holds stage st from its load until its LDS write;
  // stages go in pairs so that each set is named statically
  KvStage rs0, rs1;
  load(rs0, 0);
  load(rs1, 1);
  put(rs0, 0);
  if (nst > 2) load(rs0, 2);
  __syncthreads();
  for (int st = 0; st < nst; st += 2) {
    compute(0);
    put(rs1, 1);                              // stage st + 1 (nst is even)
    if (st + 3 < nst) load(rs1, st + 3);
    __syncthreads();
    compute(1);
    if (st + 2 < nst) {
      put(rs0, 0);
      if (st + 4 < nst) load(rs0, st + 4);
    }
    __syncthreads();
  }
  // outputs through LDS (the token buffers are free after the last barrier:
  // 8 KB a wave), so that each 128-byte row segment leaves in one piece.
  // Lane (r16, kg) of block (i, j) holds token 16 i + r16, features 16 j +
  // 4 kg .. +3 of the wave's 64 x 32 block; a row is 8 chunks of 16 bytes,
  // chunk q at q ^ ((r >> 1) & 7).
  float* out = slices == 1 ? static_cast<float*>(g.c) : ws + (int64_t)slice * g.m_len * g.c_row;
  u32x4* sc = s_a[wave >> 1] + (wave & 1) * (64 * 8);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = 16 * i + r16, q = 4 * j + kg;
      sc[r * 8 + (q ^ ((r >> 1) & 7))] = __builtin_bit_cast(u32x4, acc[i][j]);
    }
  // the reads below take other lanes' writes: a wave's LDS instructions
  // complete in order, and the compiler must not move the reads above them
  asm volatile("" ::: "memory");
  // lane L stores chunk L % 8 of rows L / 8 + 8 t: features 32 wn + 4 (L % 8) .. +3
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int r = lane / 8 + 8 * t, q = lane % 8;
    const u32x4 v = sc[r * 8 + (q ^ ((r >> 1) & 7))];
    const int m = m0 + 64 * wm + r;
    if (m < g.m_len) *reinterpret_cast<u32x4*>(out + (int64_t)m * g.c_row + n0 + 32 * wn + 4 * q) = v;
  }
}

// kv = sum over the S slices of the workspace, in slice order: thread t of
// workgroup b adds float4 number 256 b + t of every slice, loading eight
// slices at a time before adding them (one load, wait and add per slice
// made 14 slices 14 memory round trips: 5.2 us for 256 tokens)
__global__ __launch_bounds__(256) void kv_reduce_kernel(const float4* ws, float4* kv, int64_t n4, int slices) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  float4 v = ws[i];
  for (int s = 1; s < slices; s += 8) {
    float4 x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s + j < slices) x[j] = ws[(int64_t)(s + j) * n4 + i];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s + j < slices) {
        v.x += x[j].x; v.y += x[j].y; v.z += x[j].z; v.w += x[j].w;
      }
  }
  kv[i] = v;
}

template <typename TA, typename TC, int WM, int WN, int KW, int NW, int U>
hipError_t launch_gemm(const GemmParams& g, int batches, hipStream_t stream) {
  constexpr int TM = 16 * WM;
  constexpr int TN = 16 * WN;
  const dim3 grid((unsigned)(g.n_len / TN), (unsigned)((g.m_len + TM - 1) / TM), (unsigned)batches);
  hipLaunchKernelGGL((gemm_nt_kernel<TA, TC, WM, WN, KW, NW, U>), grid, dim3(64 * NW), 0, stream, g);
  return hipGetLastError();
}

// RoPE of one pair at `pos`: angle pos * base^(-2i/d) in fp64 (positions run
// to 1e5 and more, where an fp32 angle would be off by 1e-2 rad).
__device__ __forceinline__ void rope_pair(float x0, float x1, int pos, int i, int d, double base, float* y0,
                                          float* y1) {
  const double theta = pow(base, -2.0 * (double)i / (double)d);
  double sn, cs;
  sincos((double)pos * theta, &sn, &cs);
  *y0 = (float)((double)x0 * cs - (double)x1 * sn);
  *y1 = (float)((double)x0 * sn + (double)x1 * cs);
}

// OCP E4M3 code of the value nearest to v (ties to the even code), saturated
// to +-448; NaN -> 0x7F.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  if (a != a) return 0x7Fu;
  if (a >= 448.f) return sign | 0x7Eu;
  if (a < 0.015625f) return sign | (uint32_t)rintf(a * 512.f);   // subnormal steps of 2^-9 (8 = 2^-6)
  const int e = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;  // 2^e <= a < 2^(e+1), -6 <= e <= 8
  const int m = (int)rintf(ldexpf(a, 3 - e));                    // 8 .. 16
  const int code = ((e + 7) << 3) + m - 8;                       // m = 16 carries into the exponent
  return sign | (uint32_t)(code > 0x7E ? 0x7E : code);
}

// One new row per workgroup (token t = b S_q + s, position seq_len - S_q + s):
// 128 threads, thread k holds latent values 4k .. 4k + 3 (block k / 32),
// threads 0..31 the RoPE pairs.  A position outside the block table's
// capacity or a page outside the cache is skipped (nothing is written).
__global__ __launch_bounds__(128) void cache_append_kernel(AppendParams p) {
  const int t = blockIdx.x;
  const int b = t / p.s_q, s = t % p.s_q;
  const int pos = p.seq_lens[b] - p.s_q + s;
  if (pos < 0 || pos >= p.max_blocks * kPage) return;
  const int64_t entry = (int64_t)b * p.max_blocks + pos / kPage;
  const int64_t page = p.block_table ? (int64_t)p.block_table[entry] : entry;
  if (page < 0 || page >= p.num_blocks) return;
  const int64_t slot = page * kPage + (pos % kPage);
  const int tid = threadIdx.x;
  const float* row = p.kv + (int64_t)t * kRow;
  const float4 v = reinterpret_cast<const float4*>(row)[tid];
  float k0 = 0.f, k1 = 0.f;
  if (tid < kRope / 2) rope_pair(row[kLatent + 2 * tid], row[kLatent + 2 * tid + 1], pos, tid, kRope, p.base, &k0, &k1);
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  if (!p.fp8) {
    __bf16* dst = static_cast<__bf16*>(p.rows) + slot * kRow;
    bf16x4 c;
    c[0] = (__bf16)v.x;
    c[1] = (__bf16)v.y;
    c[2] = (__bf16)v.z;
    c[3] = (__bf16)v.w;
    *reinterpret_cast<bf16x4*>(dst + 4 * tid) = c;              // one 8-byte store
    if (tid < kRope / 2) {
      bf16x2 r;
      r[0] = (__bf16)k0;
      r[1] = (__bf16)k1;
      *reinterpret_cast<bf16x2*>(dst + kLatent + 2 * tid) = r;
    }
    return;
  }
  // e4m3: block amax over the 32 threads of the block (lanes 0..31 / 32..63 of a wave)
  float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
#pragma unroll
  for (int off = 16; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float sc = amax > 0.f ? __fdiv_rn(amax, 448.f) : 1.f;
  const uint32_t code = e4m3_encode(__fdiv_rn(v.x, sc)) | (e4m3_encode(__fdiv_rn(v.y, sc)) << 8) |
                        (e4m3_encode(__fdiv_rn(v.z, sc)) << 16) | (e4m3_encode(__fdiv_rn(v.w, sc)) << 24);
  reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(p.rows) + slot * kLatent)[tid] = code;
  if ((tid & 31) == 0) p.scales[slot * 4 + tid / 32] = sc;
  if (tid < kRope / 2) {
    bf16x2 r;
    r[0] = (__bf16)k0;
    r[1] = (__bf16)k1;
    *reinterpret_cast<bf16x2*>(p.rope + slot * kRope + 2 * tid) = r;
  }
}

}  // namespace

hipError_t launch_gemm_nt(const GemmParams& g, int batches, GemmKind kind, hipStream_t stream) {
  switch (kind) {
    // measured on the 256-token MTP step (HIP events around graph replays,
    // inputs rotated past the Infinity Cache): output values 20 us (a 2 x 2
    // wave grid loading its operands straight from global memory: 29 us);
    // projection 32 x 32 tiles with K over the four waves (27 us; eight
    // waves: 28 us)
    case GemmKind::kOutputAbsorb:
      if (g.k_len != kAoK || g.n_len != kAoN || batches != kHeads) return hipErrorInvalidValue;
      hipLaunchKernelGGL(absorb_output_kernel, dim3((unsigned)kHeads, (unsigned)((g.m_len + kAoTileM - 1) / kAoTileM)),
                         dim3(256), 0, stream, g);
      return hipGetLastError();
    case GemmKind::kBf16ToF32SplitK: return launch_gemm<__bf16, float, 2, 2, 4, 4, 2>(g, batches, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_kv_project_split(const GemmParams& g, float* ws, int slices, hipStream_t stream) {
  if (slices < 1 || g.n_len % kKvTileN != 0 || g.k_len % (128 * slices) != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kv_partial_kernel,
                     dim3((unsigned)((g.m_len + kKvTileM - 1) / kKvTileM), (unsigned)(g.n_len / kKvTileN), (unsigned)slices),
                     dim3(256), 0, stream, g, ws, slices);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || slices == 1) return e;
  const int64_t n4 = (int64_t)g.m_len * g.c_row / 4;
  hipLaunchKernelGGL(kv_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream,
                     reinterpret_cast<const float4*>(ws), static_cast<float4*>(g.c), n4, slices);
  return hipGetLastError();
}

hipError_t launch_query_absorb(const GemmParams& g, const RopeParams& r, hipStream_t stream) {
  if (g.k_len != kAqK || g.n_len != kAqN || r.tokens != g.m_len) return hipErrorInvalidValue;
  hipLaunchKernelGGL(absorb_query_kernel, dim3((unsigned)kHeads, (unsigned)((g.m_len + kAqTileM - 1) / kAqTileM)),
                     dim3(256), 0, stream, g, r);
  return hipGetLastError();
}

hipError_t launch_cache_append(const AppendParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(cache_append_kernel, dim3((unsigned)(p.batch * p.s_q)), dim3(128), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
