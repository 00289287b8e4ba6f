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

// Heads handled by one workgroup for a given number of query tokens.
inline int heads_per_block(int s_q) { return s_q == 1 ? 128 : 64; }

// Kernel launchers (defined next to the kernels).  They return the HIP error
// of the launch.
hipError_t launch_decode(const DecodeParams& p, int s_q, bool fp8, hipStream_t stream);
hipError_t launch_combine(const CombineParams& p, hipStream_t stream);

}  // namespace mla
