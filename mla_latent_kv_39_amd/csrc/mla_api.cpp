// The C ABI of libmla: descriptor checks on the host, then kernel launches on
// the caller's stream.  Nothing is allocated, freed or synchronised here.
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

mla_status check_device_id(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return MLA_ERR_DEVICE;
  int state = g_device_ok[dev].load(std::memory_order_relaxed);
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MLA_ERR_DEVICE;
    state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_device_ok[dev].store(state, std::memory_order_relaxed);
  }
  return state == 1 ? MLA_OK : MLA_ERR_DEVICE;
}

mla_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_DEVICE;
  return check_device_id(dev);
}

bool present(const mla_tensor* t) { return t != nullptr && t->data != nullptr; }

bool aligned16(const mla_tensor* t) { return ((uintptr_t)t->data & 15) == 0; }
bool aligned4(const mla_tensor* t) { return ((uintptr_t)t->data & 3) == 0; }

// dtype, then rank and shape (want[k] < 0: any size >= 1), then dense row-major strides
mla_status check_tensor(const mla_tensor* t, mla_dtype dtype, int rank, const int64_t* want) {
  if (!present(t)) return MLA_ERR_NULL;
  if (t->dtype != dtype) return MLA_ERR_DTYPE;
  if (t->rank != rank) return MLA_ERR_SHAPE;
  int64_t expect = 1;
  for (int k = rank - 1; k >= 0; --k) {
    const int64_t n = t->shape[k];
    if (n < 1 || (want[k] >= 0 && n != want[k])) return MLA_ERR_SHAPE;
    if (n != 1 && t->strides[k] != expect) return MLA_ERR_SHAPE;
    if (expect > ((int64_t)1 << 52) / n) return MLA_ERR_SHAPE;   // sizes far past any device memory
    expect *= n;
  }
  return MLA_OK;
}

#define MLA_TRY(x)                    \
  do {                                \
    const mla_status st_ = (x);       \
    if (st_ != MLA_OK) return st_;    \
  } while (0)

bool supported_tokens(int64_t s_q) { return s_q >= 1 && s_q <= mla::kMaxTokens; }

// The cache descriptors: kind (bf16 / e4m3), pages NB, and for a contiguous
// cache the pages per sequence.
struct CacheView {
  bool fp8 = false;
  int64_t num_blocks = 0;     // pages of 64 rows
  int64_t contig_blocks = 0;  // contiguous layout: pages per sequence
};

mla_status check_cache(const mla_latent_cache* c, bool paged, int64_t batch, CacheView* v) {
  if (c == nullptr || !present(&c->rows)) return MLA_ERR_NULL;
  const mla_tensor& r = c->rows;
  if (r.dtype == MLA_DTYPE_BF16) {
    v->fp8 = false;
  } else if (r.dtype == MLA_DTYPE_FP8_E4M3) {
    v->fp8 = true;
  } else {
    return MLA_ERR_DTYPE;
  }
  if (r.rank != 3) return MLA_ERR_SHAPE;
  const int64_t width = v->fp8 ? MLA_LATENT_DIM : MLA_ROW_DIM;
  const int64_t lead = r.shape[0], rows = r.shape[1];
  // page size: 64 rows; a contiguous cache may also come as [B, L_cap, .]
  if (paged && rows != MLA_BLOCK_SIZE) {
    return (rows > 0 && (rows & (rows - 1)) == 0) ? MLA_ERR_UNSUPPORTED : MLA_ERR_SHAPE;
  }
  if (!paged && (rows < 1 || rows % MLA_BLOCK_SIZE != 0)) return MLA_ERR_SHAPE;
  const int64_t want[3] = {-1, rows, width};
  MLA_TRY(check_tensor(&r, (mla_dtype)r.dtype, 3, want));
  v->num_blocks = lead * (rows / MLA_BLOCK_SIZE);
  if (!paged) {
    if (rows == MLA_BLOCK_SIZE) {
      if (lead % batch != 0) return MLA_ERR_SHAPE;    // [B * max_blocks, 64, .]
      v->contig_blocks = lead / batch;
    } else {
      if (lead != batch) return MLA_ERR_SHAPE;         // [B, L_cap, .]
      v->contig_blocks = rows / MLA_BLOCK_SIZE;
    }
  }
  if (v->fp8) {
    const int64_t ws[3] = {lead, rows, MLA_LATENT_DIM / MLA_FP8_GROUP};
    const int64_t wr[3] = {lead, rows, MLA_ROPE_DIM};
    MLA_TRY(check_tensor(&c->scales, MLA_DTYPE_FP32, 3, ws));
    MLA_TRY(check_tensor(&c->rope, MLA_DTYPE_BF16, 3, wr));
  }
  return MLA_OK;
}

// Split count from partial_lse (leading dimension), with both partial buffers checked.
mla_status check_partials(const mla_tensor* partial_out, const mla_tensor* partial_lse, int64_t s_q,
                          int32_t* parts) {
  if (!present(partial_lse)) {
    *parts = 1;
    return MLA_OK;    // one partition: every sequence is finished by the decode
  }
  const int64_t wl[4] = {-1, 2, s_q, MLA_NUM_HEADS};
  MLA_TRY(check_tensor(partial_lse, MLA_DTYPE_FP32, 4, wl));
  const int64_t p = partial_lse->shape[0];
  if (p > MLA_MAX_SPLITS || (p & (p - 1)) != 0) return MLA_ERR_SHAPE;   // partitions are cut with shifts
  if (p * s_q > MLA_MAX_SPLIT_TOKENS) return MLA_ERR_SHAPE;              // 32-bit row offsets in the kernels
  *parts = (int32_t)p;
  if (p == 1) return MLA_OK;
  const int64_t wo[1] = {-1};
  MLA_TRY(check_tensor(partial_out, MLA_DTYPE_UINT8, 1, wo));
  if ((size_t)partial_out->shape[0] < mla_partial_out_bytes((int32_t)p, (int32_t)s_q)) return MLA_ERR_SHAPE;
  if (((uintptr_t)partial_out->data & 15) != 0) return MLA_ERR_SHAPE;  // 16-byte stores
  return MLA_OK;
}

// Batch and query tokens from out_latent, with out_latent and lse checked.
mla_status check_outputs(const mla_tensor* out_latent, const mla_tensor* lse, int64_t* batch, int64_t* s_q) {
  if (!present(out_latent) || !present(lse)) return MLA_ERR_NULL;
  if (out_latent->dtype != MLA_DTYPE_FP32) return MLA_ERR_DTYPE;
  if (out_latent->rank != 4) return MLA_ERR_SHAPE;
  const int64_t b = out_latent->shape[0], s = out_latent->shape[1];
  if (b < 1 || s < 1) return MLA_ERR_SHAPE;
  const int64_t wo[4] = {b, s, MLA_NUM_HEADS, MLA_LATENT_DIM};
  const int64_t wl[3] = {b, s, MLA_NUM_HEADS};
  MLA_TRY(check_tensor(out_latent, MLA_DTYPE_FP32, 4, wo));
  MLA_TRY(check_tensor(lse, MLA_DTYPE_FP32, 3, wl));
  if (b > INT_MAX / 4) return MLA_ERR_SHAPE;
  if (!supported_tokens(s)) return MLA_ERR_UNSUPPORTED;
  *batch = b;
  *s_q = s;
  return MLA_OK;
}

// Everything mla_decode checks except the partials; fills p (partials unset)
// and returns S_q and the cache kind.
mla_status prepare_decode(const mla_tensor* q_absorbed, const mla_tensor* q_rope, const mla_latent_cache* cache,
                          const mla_tensor* block_table, const mla_tensor* seq_lens, float scale,
                          const mla_tensor* out_latent, const mla_tensor* lse, mla::DecodeParams* p,
                          int64_t* s_q, bool* fp8) {
  int64_t B = 0, S = 0;
  MLA_TRY(check_outputs(out_latent, lse, &B, &S));
  const int64_t wq[4] = {B, S, MLA_NUM_HEADS, MLA_LATENT_DIM};
  const int64_t wr[4] = {B, S, MLA_NUM_HEADS, MLA_ROPE_DIM};
  const int64_t wl[1] = {B};
  MLA_TRY(check_tensor(q_absorbed, MLA_DTYPE_BF16, 4, wq));
  MLA_TRY(check_tensor(q_rope, MLA_DTYPE_BF16, 4, wr));
  MLA_TRY(check_tensor(seq_lens, MLA_DTYPE_INT32, 1, wl));
  const bool paged = present(block_table);
  int64_t max_blocks = 0;
  if (paged) {
    const int64_t wt[2] = {B, -1};
    MLA_TRY(check_tensor(block_table, MLA_DTYPE_INT32, 2, wt));
    max_blocks = block_table->shape[1];
  }
  CacheView cv;
  MLA_TRY(check_cache(cache, paged, B, &cv));
  if (!paged) max_blocks = cv.contig_blocks;
  if (!std::isfinite(scale)) return MLA_ERR_SHAPE;
  // the kernels move Q, cache rows and outputs in 16-byte pieces, lengths,
  // table entries and lse in 4-byte ones
  if (!aligned16(q_absorbed) || !aligned16(q_rope) || !aligned16(out_latent) || !aligned4(lse) ||
      !aligned16(&cache->rows) || !aligned4(seq_lens) || (paged && !aligned4(block_table)))
    return MLA_ERR_SHAPE;
  if (cv.fp8 && (!aligned16(&cache->scales) || !aligned16(&cache->rope))) return MLA_ERR_SHAPE;
  // all units of the batch are counted in int32 inside the kernels
  if (max_blocks > INT_MAX / 2 || B * (max_blocks + mla::kSegWeight) > (int64_t)INT_MAX / 2) return MLA_ERR_SHAPE;
  p->q_abs = static_cast<const __bf16*>(q_absorbed->data);
  p->q_rope = static_cast<const __bf16*>(q_rope->data);
  p->rows = static_cast<const char*>(cache->rows.data);
  p->fp8_scales = cv.fp8 ? static_cast<const float*>(cache->scales.data) : nullptr;
  p->fp8_rope = cv.fp8 ? static_cast<const __bf16*>(cache->rope.data) : nullptr;
  p->block_table = paged ? static_cast<const int32_t*>(block_table->data) : nullptr;
  p->seq_lens = static_cast<const int32_t*>(seq_lens->data);
  p->out = static_cast<float*>(out_latent->data);
  p->lse = static_cast<float*>(lse->data);
  p->scale_log2 = scale * 1.4426950408889634f;
  p->max_blocks = (int32_t)max_blocks;
  p->batch = (int32_t)B;
  *s_q = S;
  *fp8 = cv.fp8;
  return MLA_OK;
}

mla::CombineParams combine_params(const mla::DecodeParams& d, int s_q) {
  mla::CombineParams p;
  p.part_out = d.part_out;
  p.part_lse = d.part_lse;
  p.seq_lens = d.seq_lens;
  p.out = d.out;
  p.lse = d.lse;
  p.batch = d.batch;
  p.s_q = s_q;
  p.num_parts = d.num_parts;
  p.log2_parts = 0;
  while ((1 << p.log2_parts) < d.num_parts) ++p.log2_parts;
  return p;
}

}  // namespace

extern "C" {

mla_status mla_decode(const mla_tensor* q_absorbed, const mla_tensor* q_rope, const mla_latent_cache* cache,
                      const mla_tensor* block_table, const mla_tensor* seq_lens, float scale,
                      const mla_tensor* out_latent, const mla_tensor* lse, const mla_tensor* partial_out,
                      const mla_tensor* partial_lse, hipStream_t stream) {
  mla::DecodeParams p;
  int64_t S = 0;
  bool fp8 = false;
  MLA_TRY(prepare_decode(q_absorbed, q_rope, cache, block_table, seq_lens, scale, out_latent, lse, &p, &S, &fp8));
  int32_t parts = 1;
  MLA_TRY(check_partials(partial_out, partial_lse, S, &parts));
  MLA_TRY(check_device());
  p.part_out = parts > 1 ? partial_out->data : nullptr;
  p.part_lse = parts > 1 ? static_cast<float*>(partial_lse->data) : nullptr;
  p.num_parts = parts;
  const hipError_t err = mla::launch_decode(p, (int)S, fp8, stream);
  return err == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

mla_status mla_decode_noalloc(const mla_tensor* q_absorbed, const mla_tensor* q_rope, const mla_latent_cache* cache,
                              const mla_tensor* block_table, const mla_tensor* seq_lens, float scale,
                              const mla_tensor* out_latent, const mla_tensor* lse, int32_t num_splits,
                              hipStream_t stream) {
  mla::DecodeParams p;
  int64_t S = 0;
  bool fp8 = false;
  MLA_TRY(prepare_decode(q_absorbed, q_rope, cache, block_table, seq_lens, scale, out_latent, lse, &p, &S, &fp8));
  if (num_splits < 1 || num_splits > MLA_MAX_SPLITS || (num_splits & (num_splits - 1)) != 0) return MLA_ERR_SHAPE;
  if ((int64_t)num_splits * S > mla::kNoallocMaxSplitTokens) return MLA_ERR_SCRATCH;
  MLA_TRY(check_device());
  void* scratch = nullptr;
  if (num_splits > 1 && mla::noalloc_scratch(&scratch) != hipSuccess) return MLA_ERR_DEVICE;
  // partial blocks and descales from the start of the scratch, partial_lse at a
  // fixed offset; every partial the combine reads is written by this decode
  p.part_out = num_splits > 1 ? scratch : nullptr;
  p.part_lse = num_splits > 1 ? reinterpret_cast<float*>(static_cast<char*>(scratch) + mla::kNoallocLseOffset)
                              : nullptr;
  p.num_parts = num_splits;
  if (mla::launch_decode(p, (int)S, fp8, stream) != hipSuccess) return MLA_ERR_LAUNCH;
  if (num_splits == 1) return MLA_OK;
  return mla::launch_combine(combine_params(p, (int)S), stream) == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

mla_status mla_combine(const mla_tensor* partial_out, const mla_tensor* partial_lse, const mla_tensor* seq_lens,
                       const mla_tensor* out_latent, const mla_tensor* lse, hipStream_t stream) {
  int64_t B = 0, S = 0;
  MLA_TRY(check_outputs(out_latent, lse, &B, &S));
  const int64_t wl[1] = {B};
  MLA_TRY(check_tensor(seq_lens, MLA_DTYPE_INT32, 1, wl));
  int32_t parts = 1;
  MLA_TRY(check_partials(partial_out, partial_lse, S, &parts));
  if (parts == 1) return MLA_OK;  // a single partition holds every sequence whole
  if (!aligned16(out_latent) || !aligned4(lse) || !aligned4(seq_lens) || !aligned4(partial_lse))
    return MLA_ERR_SHAPE;
  MLA_TRY(check_device());
  mla::CombineParams p;
  p.part_out = partial_out->data;
  p.part_lse = static_cast<const float*>(partial_lse->data);
  p.seq_lens = static_cast<const int32_t*>(seq_lens->data);
  p.out = static_cast<float*>(out_latent->data);
  p.lse = static_cast<float*>(lse->data);
  p.batch = (int32_t)B;
  p.s_q = (int32_t)S;
  p.num_parts = parts;
  p.log2_parts = 0;
  while ((1 << p.log2_parts) < parts) ++p.log2_parts;
  return mla::launch_combine(p, stream) == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

mla_status mla_absorb_query(const mla_tensor* q_c, const mla_tensor* q_r, const mla_tensor* w_uk_t,
                            const mla_tensor* seq_lens, float rope_base, const mla_tensor* q_absorbed,
                            const mla_tensor* q_rope, hipStream_t stream) {
  if (!present(q_c)) return MLA_ERR_NULL;
  if (q_c->dtype != MLA_DTYPE_BF16) return MLA_ERR_DTYPE;
  if (q_c->rank != 4) return MLA_ERR_SHAPE;
  const int64_t B = q_c->shape[0], S = q_c->shape[1];
  const int64_t wc[4] = {B, S, MLA_NUM_HEADS, MLA_HEAD_DIM};
  const int64_t wr[4] = {B, S, MLA_NUM_HEADS, MLA_ROPE_DIM};
  const int64_t ww[3] = {MLA_NUM_HEADS, MLA_LATENT_DIM, MLA_HEAD_DIM};
  const int64_t wa[4] = {B, S, MLA_NUM_HEADS, MLA_LATENT_DIM};
  const int64_t wl[1] = {B};
  MLA_TRY(check_tensor(q_c, MLA_DTYPE_BF16, 4, wc));
  MLA_TRY(check_tensor(q_r, MLA_DTYPE_BF16, 4, wr));
  MLA_TRY(check_tensor(w_uk_t, MLA_DTYPE_BF16, 3, ww));
  MLA_TRY(check_tensor(seq_lens, MLA_DTYPE_INT32, 1, wl));
  MLA_TRY(check_tensor(q_absorbed, MLA_DTYPE_BF16, 4, wa));
  MLA_TRY(check_tensor(q_rope, MLA_DTYPE_BF16, 4, wr));
  if (!(std::isfinite(rope_base) && rope_base > 0.f)) return MLA_ERR_SHAPE;
  if (B * S > INT_MAX / (MLA_NUM_HEADS * MLA_LATENT_DIM)) return MLA_ERR_SHAPE;
  if (!aligned16(q_c) || !aligned16(w_uk_t) || !aligned16(q_absorbed) || !aligned16(q_r) || !aligned16(q_rope))
    return MLA_ERR_SHAPE;
  MLA_TRY(check_device());
  mla::GemmParams g;
  g.a = q_c->data;
  g.w = static_cast<const __bf16*>(w_uk_t->data);
  g.c = q_absorbed->data;
  g.a_batch = MLA_HEAD_DIM;                    // head h of a token row
  g.a_row = (int64_t)MLA_NUM_HEADS * MLA_HEAD_DIM;
  g.w_batch = (int64_t)MLA_LATENT_DIM * MLA_HEAD_DIM;
  g.c_batch = MLA_LATENT_DIM;
  g.c_row = (int64_t)MLA_NUM_HEADS * MLA_LATENT_DIM;
  g.m_len = (int32_t)(B * S);
  g.n_len = MLA_LATENT_DIM;
  g.k_len = MLA_HEAD_DIM;
  mla::RopeParams r;
  r.src = static_cast<const __bf16*>(q_r->data);
  r.dst = static_cast<__bf16*>(q_rope->data);
  r.seq_lens = static_cast<const int32_t*>(seq_lens->data);
  r.tokens = (int32_t)(B * S);
  r.s_q = (int32_t)S;
  r.base = rope_base;
  return mla::launch_query_absorb(g, r, stream) == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

mla_status mla_absorb_output(const mla_tensor* out_latent, const mla_tensor* w_uv, const mla_tensor* out_values,
                             hipStream_t stream) {
  if (!present(out_latent)) return MLA_ERR_NULL;
  if (out_latent->dtype != MLA_DTYPE_FP32) return MLA_ERR_DTYPE;
  if (out_latent->rank != 4) return MLA_ERR_SHAPE;
  const int64_t B = out_latent->shape[0], S = out_latent->shape[1];
  const int64_t wo[4] = {B, S, MLA_NUM_HEADS, MLA_LATENT_DIM};
  const int64_t ww[3] = {MLA_NUM_HEADS, MLA_HEAD_DIM, MLA_LATENT_DIM};
  const int64_t wv[4] = {B, S, MLA_NUM_HEADS, MLA_HEAD_DIM};
  MLA_TRY(check_tensor(out_latent, MLA_DTYPE_FP32, 4, wo));
  MLA_TRY(check_tensor(w_uv, MLA_DTYPE_BF16, 3, ww));
  MLA_TRY(check_tensor(out_values, MLA_DTYPE_FP32, 4, wv));
  if (B * S > INT_MAX / (MLA_NUM_HEADS * MLA_LATENT_DIM)) return MLA_ERR_SHAPE;
  if (!aligned16(out_latent) || !aligned16(w_uv) || !aligned16(out_values)) return MLA_ERR_SHAPE;
  MLA_TRY(check_device());
  mla::GemmParams g;
  g.a = out_latent->data;
  g.w = static_cast<const __bf16*>(w_uv->data);
  g.c = out_values->data;
  g.a_batch = MLA_LATENT_DIM;
  g.a_row = (int64_t)MLA_NUM_HEADS * MLA_LATENT_DIM;
  g.w_batch = (int64_t)MLA_HEAD_DIM * MLA_LATENT_DIM;
  g.c_batch = MLA_HEAD_DIM;
  g.c_row = (int64_t)MLA_NUM_HEADS * MLA_HEAD_DIM;
  g.m_len = (int32_t)(B * S);
  g.n_len = MLA_HEAD_DIM;
  g.k_len = MLA_LATENT_DIM;
  return mla::launch_gemm_nt(g, MLA_NUM_HEADS, mla::GemmKind::kOutputAbsorb, stream) == hipSuccess
             ? MLA_OK : MLA_ERR_LAUNCH;
}

mla_status mla_kv_project(const mla_tensor* hidden, const mla_tensor* w_kv, const mla_tensor* kv,
                          hipStream_t stream) {
  if (!present(hidden)) return MLA_ERR_NULL;
  if (hidden->dtype != MLA_DTYPE_BF16) return MLA_ERR_DTYPE;
  if (hidden->rank != 2) return MLA_ERR_SHAPE;
  const int64_t T = hidden->shape[0], D = hidden->shape[1];
  const int64_t wh[2] = {T, D};
  const int64_t ww[2] = {MLA_ROW_DIM, D};
  const int64_t wk[2] = {T, MLA_ROW_DIM};
  MLA_TRY(check_tensor(hidden, MLA_DTYPE_BF16, 2, wh));
  MLA_TRY(check_tensor(w_kv, MLA_DTYPE_BF16, 2, ww));
  MLA_TRY(check_tensor(kv, MLA_DTYPE_FP32, 2, wk));
  if (D % 128 != 0 || D > (1 << 20) || T > INT_MAX / MLA_ROW_DIM) return MLA_ERR_SHAPE;
  if (!aligned16(hidden) || !aligned16(w_kv) || !aligned16(kv)) return MLA_ERR_SHAPE;
  MLA_TRY(check_device());
  mla::GemmParams g;
  g.a = hidden->data;
  g.w = static_cast<const __bf16*>(w_kv->data);
  g.c = kv->data;
  g.a_batch = g.w_batch = g.c_batch = 0;
  g.a_row = D;
  g.c_row = MLA_ROW_DIM;
  g.m_len = (int32_t)T;
  g.n_len = MLA_ROW_DIM;
  g.k_len = (int32_t)D;
  return mla::launch_gemm_nt(g, 1, mla::GemmKind::kBf16ToF32SplitK, stream) == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

int32_t mla_kv_project_splits(int64_t tokens, int64_t d) {
  if (tokens < 1 || d < 128 || d % 128 != 0 || d > (1 << 20)) return 0;
  // the most slices (a divisor of d / 128) that keep the workgroups, 64-feature
  // x 128-token tiles times slices, within one per compute unit of 256
  const int64_t tiles = ((tokens + 127) / 128) * (MLA_ROW_DIM / 64);
  int32_t best = 1;
  for (int64_t s = 1; s <= d / 128; ++s)
    if ((d / 128) % s == 0 && tiles * s <= 256) best = (int32_t)s;
  return best;
}

mla_status mla_kv_project_split(const mla_tensor* hidden, const mla_tensor* w_kv, const mla_tensor* kv,
                                const mla_tensor* workspace, hipStream_t stream) {
  if (!present(hidden) || !present(workspace)) return MLA_ERR_NULL;
  if (hidden->dtype != MLA_DTYPE_BF16) return MLA_ERR_DTYPE;
  if (hidden->rank != 2 || workspace->rank != 3) return MLA_ERR_SHAPE;
  const int64_t T = hidden->shape[0], D = hidden->shape[1], S = workspace->shape[0];
  const int64_t wh[2] = {T, D};
  const int64_t ww[2] = {MLA_ROW_DIM, D};
  const int64_t wk[2] = {T, MLA_ROW_DIM};
  const int64_t wws[3] = {S, T, MLA_ROW_DIM};
  MLA_TRY(check_tensor(hidden, MLA_DTYPE_BF16, 2, wh));
  MLA_TRY(check_tensor(w_kv, MLA_DTYPE_BF16, 2, ww));
  MLA_TRY(check_tensor(kv, MLA_DTYPE_FP32, 2, wk));
  MLA_TRY(check_tensor(workspace, MLA_DTYPE_FP32, 3, wws));
  if (D % 128 != 0 || D > (1 << 20) || T > INT_MAX / MLA_ROW_DIM) return MLA_ERR_SHAPE;
  if (S < 1 || (D / 128) % S != 0) return MLA_ERR_SHAPE;
  if ((T + 127) / 128 > 65535) return MLA_ERR_SHAPE;
  if (!aligned16(hidden) || !aligned16(w_kv) || !aligned16(kv) || !aligned16(workspace)) return MLA_ERR_SHAPE;
  MLA_TRY(check_device());
  mla::GemmParams g;
  g.a = hidden->data;
  g.w = static_cast<const __bf16*>(w_kv->data);
  g.c = kv->data;
  g.a_batch = g.w_batch = g.c_batch = 0;
  g.a_row = D;
  g.c_row = MLA_ROW_DIM;
  g.m_len = (int32_t)T;
  g.n_len = MLA_ROW_DIM;
  g.k_len = (int32_t)D;
  return mla::launch_kv_project_split(g, static_cast<float*>(workspace->data), (int)S, stream) == hipSuccess
             ? MLA_OK : MLA_ERR_LAUNCH;
}

mla_status mla_cache_append(const mla_tensor* kv, const mla_tensor* seq_lens, const mla_tensor* block_table,
                            const mla_latent_cache* cache, float rope_base, hipStream_t stream) {
  if (!present(kv)) return MLA_ERR_NULL;
  if (kv->dtype != MLA_DTYPE_FP32) return MLA_ERR_DTYPE;
  if (kv->rank != 3) return MLA_ERR_SHAPE;
  const int64_t B = kv->shape[0], S = kv->shape[1];
  const int64_t wk[3] = {B, S, MLA_ROW_DIM};
  const int64_t wl[1] = {B};
  MLA_TRY(check_tensor(kv, MLA_DTYPE_FP32, 3, wk));
  MLA_TRY(check_tensor(seq_lens, MLA_DTYPE_INT32, 1, wl));
  const bool paged = present(block_table);
  int64_t max_blocks = 0;
  if (paged) {
    const int64_t wt[2] = {B, -1};
    MLA_TRY(check_tensor(block_table, MLA_DTYPE_INT32, 2, wt));
    max_blocks = block_table->shape[1];
  }
  CacheView cv;
  MLA_TRY(check_cache(cache, paged, B, &cv));
  if (!paged) max_blocks = cv.contig_blocks;
  if (!(std::isfinite(rope_base) && rope_base > 0.f)) return MLA_ERR_SHAPE;
  if (B * S > INT_MAX || max_blocks > INT_MAX / 128) return MLA_ERR_SHAPE;
  if (!aligned16(kv) || !aligned16(&cache->rows) || !aligned4(seq_lens) || (paged && !aligned4(block_table)))
    return MLA_ERR_SHAPE;
  if (cv.fp8 && (!aligned4(&cache->scales) || !aligned4(&cache->rope))) return MLA_ERR_SHAPE;
  MLA_TRY(check_device());
  mla::AppendParams p;
  p.kv = static_cast<const float*>(kv->data);
  p.seq_lens = static_cast<const int32_t*>(seq_lens->data);
  p.block_table = paged ? static_cast<const int32_t*>(block_table->data) : nullptr;
  p.rows = cache->rows.data;
  p.scales = cv.fp8 ? static_cast<float*>(cache->scales.data) : nullptr;
  p.rope = cv.fp8 ? static_cast<__bf16*>(cache->rope.data) : nullptr;
  p.num_blocks = cv.num_blocks;
  p.max_blocks = (int32_t)max_blocks;
  p.batch = (int32_t)B;
  p.s_q = (int32_t)S;
  p.fp8 = cv.fp8 ? 1 : 0;
  p.base = rope_base;
  return mla::launch_cache_append(p, stream) == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

mla_status mla_check_indices(const mla_latent_cache* cache, const mla_tensor* block_table,
                             const mla_tensor* seq_lens, const mla_tensor* counts, hipStream_t stream) {
  if (!present(seq_lens)) return MLA_ERR_NULL;
  if (seq_lens->dtype != MLA_DTYPE_INT32) return MLA_ERR_DTYPE;
  if (seq_lens->rank != 1) return MLA_ERR_SHAPE;
  const int64_t B = seq_lens->shape[0];
  const int64_t wl[1] = {B};
  MLA_TRY(check_tensor(seq_lens, MLA_DTYPE_INT32, 1, wl));
  if (B > INT_MAX / 4) return MLA_ERR_SHAPE;
  const bool paged = present(block_table);
  int64_t max_blocks = 0;
  if (paged) {
    const int64_t wt[2] = {B, -1};
    MLA_TRY(check_tensor(block_table, MLA_DTYPE_INT32, 2, wt));
    max_blocks = block_table->shape[1];
  }
  CacheView cv;
  MLA_TRY(check_cache(cache, paged, B, &cv));
  if (!paged) max_blocks = cv.contig_blocks;
  if (max_blocks > INT_MAX / 128) return MLA_ERR_SHAPE;
  const int64_t wc[1] = {2};
  MLA_TRY(check_tensor(counts, MLA_DTYPE_INT32, 1, wc));
  if (!aligned4(seq_lens) || !aligned4(counts) || (paged && !aligned4(block_table))) return MLA_ERR_SHAPE;
  MLA_TRY(check_device());
  mla::CheckParams p;
  p.block_table = paged ? static_cast<const int32_t*>(block_table->data) : nullptr;
  p.seq_lens = static_cast<const int32_t*>(seq_lens->data);
  p.counts = static_cast<int32_t*>(counts->data);
  p.num_blocks = cv.num_blocks;
  p.max_blocks = (int32_t)max_blocks;
  p.batch = (int32_t)B;
  return mla::launch_check_indices(p, stream) == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

mla_status mla_init(int32_t device) {
  MLA_TRY(check_device_id(device));
  int prev = -1;
  if (hipGetDevice(&prev) != hipSuccess) return MLA_ERR_DEVICE;
  if (prev != device && hipSetDevice(device) != hipSuccess) return MLA_ERR_DEVICE;
  // with `device` current: the decode code object and the address of the
  // static scratch of mla_decode_noalloc on this device
  hipError_t err = mla::load_decode_module();
  void* scratch = nullptr;
  if (err == hipSuccess) err = mla::noalloc_scratch(&scratch);
  if (prev != device) (void)hipSetDevice(prev);
  return err == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

int32_t mla_num_splits_hint(int32_t device, int32_t batch, int32_t s_q, int32_t max_blocks_per_seq) {
  if (batch < 1 || !supported_tokens(s_q)) return 0;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus < 1) return 0;
  // a partition takes as many workgroups (128 query rows each) as its largest token group
  const int parts = cus / mla::token_group(s_q);
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
    case MLA_ERR_NULL: return "a required tensor or its data pointer is NULL";
    case MLA_ERR_DTYPE: return "a tensor has the wrong element type";
    case MLA_ERR_SHAPE: return "inconsistent or out-of-range shapes or strides";
    case MLA_ERR_UNSUPPORTED: return "valid request not implemented by this build";
    case MLA_ERR_LAUNCH: return "kernel launch failed";
    case MLA_ERR_DEVICE: return "current device is not gfx950 or cannot be queried";
    case MLA_ERR_SCRATCH: return "num_splits * s_q exceeds the static scratch of mla_decode_noalloc (256)";
  }
  return "unknown status";
}

int32_t mla_version(void) { return 30300; }  // 3.3.0: + the KV projection split over K

}  // extern "C"
