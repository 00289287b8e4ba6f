// The C ABI of libmla: argument checks on the host, then kernel launches on the
// caller's stream.  Nothing is allocated, freed or synchronised here.
#include <atomic>
#include <climits>
#include <cmath>
#include <cstring>

#include "../../include/mla.h"
#include "mla_internal.h"
#include "mla_schedule.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

mla_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_DEVICE;
  int state = g_device_ok[dev].load(std::memory_order_relaxed);
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MLA_ERR_DEVICE;
    state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_device_ok[dev].store(state, std::memory_order_relaxed);
  }
  return state == 1 ? MLA_OK : MLA_ERR_DEVICE;
}

mla_status check_common(int32_t batch, int32_t s_q, int32_t num_splits, const void* partial_out,
                        const float* partial_lse) {
  if (batch < 1 || s_q < 1 || num_splits < 1 || num_splits > MLA_MAX_SPLITS) return MLA_ERR_SHAPE;
  if ((num_splits & (num_splits - 1)) != 0) return MLA_ERR_SHAPE;  // partitions are cut with shifts
  if (s_q > 2) return MLA_ERR_UNSUPPORTED;
  if (num_splits > 1 && (partial_out == nullptr || partial_lse == nullptr)) return MLA_ERR_NULL;
  if (num_splits > 1 && ((uintptr_t)partial_out & 15) != 0) return MLA_ERR_SHAPE;  // 16-byte stores
  // every output index must fit the kernels' size_t arithmetic with room to spare
  const double out_elems = (double)batch * s_q * MLA_NUM_HEADS * MLA_LATENT_DIM;
  if (out_elems > 9.0e15) return MLA_ERR_SHAPE;
  return MLA_OK;
}

}  // namespace

extern "C" {

mla_status mla_decode(const void* q_absorbed, const void* q_rope, const mla_latent_cache* cache,
                      const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                      int32_t batch, int32_t s_q, float scale, int32_t num_splits, void* partial_out,
                      float* partial_lse, float* out_latent, float* lse, hipStream_t stream) {
  if (!q_absorbed || !q_rope || !cache || !seq_lens || !out_latent || !lse) return MLA_ERR_NULL;
  if (!cache->rows) return MLA_ERR_NULL;
  mla_status st = check_common(batch, s_q, num_splits, partial_out, partial_lse);
  if (st != MLA_OK) return st;
  if (cache->dtype != MLA_CACHE_BF16 && cache->dtype != MLA_CACHE_FP8_E4M3) return MLA_ERR_DTYPE;
  if (cache->dtype == MLA_CACHE_FP8_E4M3 && (!cache->scales || !cache->rope)) return MLA_ERR_NULL;
  if (cache->block_size != MLA_BLOCK_SIZE) {
    const int bs = cache->block_size;
    return (bs > 0 && (bs & (bs - 1)) == 0) ? MLA_ERR_UNSUPPORTED : MLA_ERR_SHAPE;
  }
  if (max_blocks_per_seq < 1 || cache->num_blocks < 1) return MLA_ERR_SHAPE;
  // all units of the batch are counted in int32 inside the kernels
  if ((int64_t)batch * max_blocks_per_seq > (int64_t)INT_MAX / 2) return MLA_ERR_SHAPE;
  if (block_table == nullptr && cache->num_blocks < (int64_t)batch * max_blocks_per_seq) return MLA_ERR_SHAPE;
  if (!std::isfinite(scale)) return MLA_ERR_SHAPE;
  st = check_device();
  if (st != MLA_OK) return st;

  mla::DecodeParams p;
  p.q_abs = static_cast<const __bf16*>(q_absorbed);
  p.q_rope = static_cast<const __bf16*>(q_rope);
  p.rows = static_cast<const char*>(cache->rows);
  p.fp8_scales = cache->scales;
  p.fp8_rope = static_cast<const __bf16*>(cache->rope);
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.part_out = partial_out;
  p.part_lse = partial_lse;
  p.out = out_latent;
  p.lse = lse;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.max_blocks = max_blocks_per_seq;
  p.batch = batch;
  p.num_parts = num_splits;
  const hipError_t err = mla::launch_decode(p, s_q, cache->dtype == MLA_CACHE_FP8_E4M3, stream);
  return err == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

mla_status mla_combine(const void* partial_out, const float* partial_lse, const int32_t* seq_lens,
                       int32_t batch, int32_t s_q, int32_t num_splits, float* out_latent, float* lse,
                       hipStream_t stream) {
  if (!seq_lens || !out_latent || !lse) return MLA_ERR_NULL;
  mla_status st = check_common(batch, s_q, num_splits, partial_out, partial_lse);
  if (st != MLA_OK) return st;
  if (num_splits == 1) return MLA_OK;  // a single partition holds every sequence whole
  st = check_device();
  if (st != MLA_OK) return st;
  mla::CombineParams p;
  p.part_out = partial_out;
  p.part_lse = partial_lse;
  p.seq_lens = seq_lens;
  p.out = out_latent;
  p.lse = lse;
  p.batch = batch;
  p.s_q = s_q;
  p.num_parts = num_splits;
  p.log2_parts = 0;
  while ((1 << p.log2_parts) < num_splits) ++p.log2_parts;
  return mla::launch_combine(p, stream) == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

int32_t mla_num_splits_hint(int32_t device, int32_t batch, int32_t s_q, int32_t max_blocks_per_seq) {
  if (batch < 1 || s_q < 1 || s_q > 2) return 0;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus < 1) return 0;
  int parts = s_q == 1 ? cus : cus / 2;
  int p2 = 1;
  while (p2 * 2 <= parts) p2 *= 2;  // partitions must be a power of two
  if (max_blocks_per_seq > 0) {
    // the most weighted units the partition map can see (see mla_schedule.h)
    const long long most = (long long)batch * (max_blocks_per_seq + mla::kSegWeight);
    while (p2 > 1 && most < 4LL * p2) p2 /= 2;
  }
  return p2;
}

size_t mla_partial_out_bytes(int32_t num_splits, int32_t s_q) {
  if (num_splits < 1 || s_q < 1) return 0;
  return (size_t)num_splits * 2 * s_q * (mla::kPartBlockBytes + mla::kPartDescBytes);
}

size_t mla_partial_lse_bytes(int32_t num_splits, int32_t s_q) {
  if (num_splits < 1 || s_q < 1) return 0;
  return (size_t)num_splits * 2 * s_q * MLA_NUM_HEADS * sizeof(float);
}

const char* mla_status_string(mla_status status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "a required pointer is NULL";
    case MLA_ERR_DTYPE: return "unsupported cache dtype";
    case MLA_ERR_SHAPE: return "inconsistent or out-of-range sizes";
    case MLA_ERR_UNSUPPORTED: return "valid request not implemented by this build";
    case MLA_ERR_LAUNCH: return "kernel launch failed";
    case MLA_ERR_DEVICE: return "current device is not gfx950 or cannot be queried";
  }
  return "unknown status";
}

int32_t mla_version(void) { return 200; }  // 0.2.0: fp16 partials with descales

}  // extern "C"
