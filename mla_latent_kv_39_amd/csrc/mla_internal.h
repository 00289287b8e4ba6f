// Internal declarations shared by the host API and the kernels of libmla.
#pragma once
#include <stdint.h>
#include <hip/hip_runtime.h>

namespace mla {

constexpr int kHeads = 128;
constexpr int kLatent = 512;
constexpr int kRope = 64;
constexpr int kRow = 576;
constexpr int kPage = 64;          // rows per cache page = rows per work unit
constexpr int kRowBytesBf16 = kRow * 2;  // 1152
// A partial block (split, slot, query token): 128 x 512 fp16 values; after all
// blocks, 4 x 128 fp32 descales per block (column quarter, head).
constexpr size_t kPartBlockBytes = (size_t)kHeads * kLatent * 2;
constexpr size_t kPartDescBytes = (size_t)4 * kHeads * 4;

// Everything one decode launch needs; all pointers are device pointers.
struct DecodeParams {
  const __bf16* q_abs;       // [B, S_q, 128, 512]
  const __bf16* q_rope;      // [B, S_q, 128, 64]
  const char* rows;          // bf16 pages [NB, 64, 576] or e4m3 pages [NB, 64, 512]
  const float* fp8_scales;   // [NB, 64, 4]
  const __bf16* fp8_rope;    // [NB, 64, 64]
  const int32_t* block_table;  // [B, max_blocks] or nullptr (contiguous)
  const int32_t* seq_lens;   // [B]
  void* part_out;            // P * 2 * S_q blocks of 128 x 512 fp16, then their descales
  float* part_lse;           // [P, 2, S_q, 128]
  float* out;                // [B, S_q, 128, 512]
  float* lse;                // [B, S_q, 128]
  float scale_log2;          // scale * log2(e)
  int32_t max_blocks;
  int32_t batch;
  int32_t num_parts;         // work partitions P
};

struct CombineParams {
  const void* part_out;
  const float* part_lse;
  const int32_t* seq_lens;
  float* out;
  float* lse;
  int32_t batch;
  int32_t s_q;
  int32_t num_parts;
  int32_t log2_parts;        // num_parts is a power of two
};

// Heads handled by one workgroup for a group of 1, 2 or 4 query tokens: a
// workgroup always holds 128 query rows, four waves of 32 rows of one token
// each.
inline int heads_per_block(int group) { return kHeads / group; }

// The size of the next token group when `left` tokens remain: 4, 2 or 1.
inline int token_group(int left) { return left >= 4 ? 4 : (left >= 2 ? 2 : 1); }

// Most query tokens per sequence a decode call takes (several draft tokens of
// speculative decoding; every group of up to four re-reads the rows).
constexpr int kMaxTokens = 64;

// Kernel launchers (defined next to the kernels).  They return the HIP error
// of the launch.
hipError_t launch_decode(const DecodeParams& p, int s_q, bool fp8, hipStream_t stream);
hipError_t launch_combine(const CombineParams& p, hipStream_t stream);

// Index contract of the decode (seq_lens and block_table contents).
struct CheckParams {
  const int32_t* block_table;  // [B, max_blocks] or nullptr (contiguous)
  const int32_t* seq_lens;     // [B]
  int32_t* counts;             // [2]: bad lengths, bad table entries
  int64_t num_blocks;
  int32_t max_blocks;
  int32_t batch;
};
hipError_t launch_check_indices(const CheckParams& p, hipStream_t stream);

// C[M x N] = A[M x K] W[N x K]^T per batch (mla_proj.hip): element offsets
// A (m, k) = z a_batch + m a_row + k, W (n, k) = z w_batch + n k_len + k,
// C (m, n) = z c_batch + m c_row + n.  k_len % 128 == 0; the output
// absorption takes K = 512, N = 128 per head, the query absorption K = 128,
// N = 512 per head, the projection n_len a multiple of 32; 16-byte aligned
// A, W and C rows.
struct GemmParams {
  const void* a;
  const __bf16* w;
  void* c;
  int64_t a_batch, a_row, w_batch, c_batch, c_row;
  int32_t m_len, n_len, k_len;
};
enum class GemmKind {
  kOutputAbsorb,    // fp32 A (rounded to bf16 when used), fp32 C, K = 512, N = 128 per head
  kBf16ToF32SplitK  // bf16 A, fp32 C, 32 x 32 tiles, K split over the four waves
};
hipError_t launch_gemm_nt(const GemmParams& g, int batches, GemmKind kind, hipStream_t stream);

// The KV projection with K cut into `slices` (a divisor of k_len / 128):
// partial sums into ws [slices, m_len, n_len] (fp32; c_row == n_len), then
// their sum in slice order into C.  slices == 1 writes C directly.
hipError_t launch_kv_project_split(const GemmParams& g, float* ws, int slices, hipStream_t stream);

// RoPE of the query's q^R: [tokens = B S_q, 128, 64] bf16 -> bf16, position
// seq_len[b] - S_q + s of token b S_q + s.
struct RopeParams {
  const __bf16* src;
  __bf16* dst;
  const int32_t* seq_lens;
  int32_t tokens;
  int32_t s_q;
  double base;
};
// The absorbed query (g: A = q^C, W = W^UK^T per head, C = q_absorbed; K = 128,
// N = 512, 128 heads) and the RoPE of q^R (r), in one launch.
hipError_t launch_query_absorb(const GemmParams& g, const RopeParams& r, hipStream_t stream);

// New cache rows: kv [B S_q, 576] fp32 ([c^KV ; k^R before RoPE]) -> the page
// slot of position seq_len[b] - S_q + s, bf16 rows or the e4m3 bundle.
struct AppendParams {
  const float* kv;
  const int32_t* seq_lens;
  const int32_t* block_table;   // [B, max_blocks] or nullptr (contiguous)
  void* rows;                   // bf16 [NB, 64, 576] or e4m3 [NB, 64, 512]
  float* scales;                // e4m3: [NB, 64, 4]
  __bf16* rope;                 // e4m3: [NB, 64, 64]
  int64_t num_blocks;
  int32_t max_blocks;
  int32_t batch;
  int32_t s_q;
  int32_t fp8;
  double base;
};
hipError_t launch_cache_append(const AppendParams& p, hipStream_t stream);

// Load the decode code object on the current device (idempotent).
hipError_t load_decode_module();

// mla_decode_noalloc: the largest num_splits * s_q its static scratch holds,
// and the scratch bytes (partial_out blocks and descales, then partial_lse).
constexpr int kNoallocMaxSplitTokens = 256;
constexpr size_t kNoallocLseOffset = (size_t)kNoallocMaxSplitTokens * 2 * (kPartBlockBytes + kPartDescBytes);
constexpr size_t kNoallocScratchBytes = kNoallocLseOffset + (size_t)kNoallocMaxSplitTokens * 2 * kHeads * 4;
static_assert(kNoallocScratchBytes == 68419584, "MLA_NOALLOC_SCRATCH_BYTES");
// The current device's address of the static scratch (taken once per device).
hipError_t noalloc_scratch(void** ptr);

}  // namespace mla
