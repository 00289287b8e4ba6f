// The host side of libmla's C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer, on the CPU.  The HIP runtime calls and the
// kernel launchers are replaced by recording stubs (a gfx950 device 0 with 256
// compute units, launches that succeed), so every entry point runs its
// descriptor checks and its launch-parameter arithmetic here: directed cases
// (each argument of a valid call broken in turn: the status it must give),
// then random descriptors (any dtype, rank, shape, stride and pointer; only a
// status may come back, never a sanitizer report or a launch).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <random>

#include "../../include/mla.h"
#include "../../mla_latent_kv_39_amd/csrc/mla_internal.h"

namespace {
int g_fail = 0;
int g_decode_launches = 0, g_combine_launches = 0, g_gemm_launches = 0, g_other_launches = 0;
mla::DecodeParams g_decode{};
int g_decode_sq = 0;
bool g_decode_fp8 = false;
mla::CombineParams g_combine{};

#define EXPECT(cond, ...)                                    \
  do {                                                       \
    if (!(cond)) {                                           \
      std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      std::fprintf(stderr, __VA_ARGS__);                     \
      std::fprintf(stderr, "\n");                            \
      ++g_fail;                                              \
    }                                                        \
  } while (0)
}  // namespace

// ---------------------------------------------------------------- stubs
namespace mla {
hipError_t launch_decode(const DecodeParams& p, int s_q, bool fp8, hipStream_t) {
  ++g_decode_launches;
  g_decode = p;
  g_decode_sq = s_q;
  g_decode_fp8 = fp8;
  return hipSuccess;
}
hipError_t launch_combine(const CombineParams& p, hipStream_t) {
  ++g_combine_launches;
  g_combine = p;
  return hipSuccess;
}
hipError_t launch_check_indices(const CheckParams&, hipStream_t) { ++g_other_launches; return hipSuccess; }
hipError_t launch_gemm_nt(const GemmParams&, int, GemmKind, hipStream_t) { ++g_gemm_launches; return hipSuccess; }
hipError_t launch_query_absorb(const GemmParams&, const RopeParams&, hipStream_t) { ++g_gemm_launches; return hipSuccess; }
hipError_t launch_kv_project_split(const GemmParams&, float*, int, hipStream_t) { ++g_gemm_launches; return hipSuccess; }
hipError_t launch_cache_append(const AppendParams&, hipStream_t) { ++g_other_launches; return hipSuccess; }
hipError_t load_decode_module() { return hipSuccess; }
hipError_t noalloc_scratch(void** ptr) {
  *ptr = reinterpret_cast<void*>(uintptr_t(0x7f0000000000));   // never dereferenced on the host
  return hipSuccess;
}
}  // namespace mla

hipError_t hipGetDevice(int* device) { *device = 0; return hipSuccess; }
hipError_t hipSetDevice(int) { return hipSuccess; }
hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t, int) { *value = 256; return hipSuccess; }
hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600* prop, int device) {
  std::memset(prop, 0, sizeof(*prop));
  if (device != 0) return hipErrorInvalidDevice;
  std::strcpy(prop->gcnArchName, "gfx950:sramecc+:xnack-");
  return hipSuccess;
}

// ---------------------------------------------------------------- descriptors
namespace {
uintptr_t g_next_ptr = 0x10000;
void* fake_ptr() {  // distinct, 256-byte aligned, never dereferenced
  g_next_ptr += 0x100000;
  return reinterpret_cast<void*>(g_next_ptr);
}

mla_tensor dense(mla_dtype dt, std::initializer_list<int64_t> shape) {
  mla_tensor t{};
  t.data = fake_ptr();
  t.dtype = dt;
  t.rank = (int32_t)shape.size();
  int k = 0;
  for (int64_t n : shape) t.shape[k++] = n;
  int64_t s = 1;
  for (int j = t.rank - 1; j >= 0; --j) {
    t.strides[j] = s;
    s *= t.shape[j];
  }
  return t;
}

struct DecodeCall {
  mla_tensor q, qr, table, lens, out, lse, pout, plse;
  mla_latent_cache cache{};
  float scale = 1.0f / std::sqrt(192.0f);
  DecodeCall(int64_t B, int64_t S, int64_t P, bool fp8, bool paged, int64_t nb = 40, int64_t mb = 8) {
    q = dense(MLA_DTYPE_BF16, {B, S, 128, 512});
    qr = dense(MLA_DTYPE_BF16, {B, S, 128, 64});
    table = paged ? dense(MLA_DTYPE_INT32, {B, mb}) : mla_tensor{};
    lens = dense(MLA_DTYPE_INT32, {B});
    out = dense(MLA_DTYPE_FP32, {B, S, 128, 512});
    lse = dense(MLA_DTYPE_FP32, {B, S, 128});
    if (P > 1) {
      pout = dense(MLA_DTYPE_UINT8, {(int64_t)mla_partial_out_bytes((int32_t)P, (int32_t)S)});
      plse = dense(MLA_DTYPE_FP32, {P, 2, S, 128});
    } else {
      pout = mla_tensor{};
      plse = mla_tensor{};
    }
    const int64_t pages = paged ? nb : B * mb;
    if (fp8) {
      cache.rows = dense(MLA_DTYPE_FP8_E4M3, {pages, 64, 512});
      cache.scales = dense(MLA_DTYPE_FP32, {pages, 64, 4});
      cache.rope = dense(MLA_DTYPE_BF16, {pages, 64, 64});
    } else {
      cache.rows = dense(MLA_DTYPE_BF16, {pages, 64, 576});
    }
  }
  mla_status run() {
    return mla_decode(&q, &qr, &cache, table.data ? &table : nullptr, &lens, scale, &out, &lse,
                      pout.data ? &pout : nullptr, plse.data ? &plse : nullptr, nullptr);
  }
};

void directed_decode() {
  // valid calls, with the launch parameters they derive
  for (bool fp8 : {false, true})
    for (bool paged : {false, true})
      for (int64_t S : {1, 2, 5, 64})
        for (int64_t P : {1, 4, 256}) {
          DecodeCall c(3, S, P, fp8, paged);
          const int before = g_decode_launches;
          const mla_status st = c.run();
          EXPECT(st == MLA_OK, "valid decode fp8=%d paged=%d S=%lld P=%lld: status %d", fp8, paged,
                 (long long)S, (long long)P, st);
          EXPECT(g_decode_launches == before + 1, "one launch per decode call");
          EXPECT(g_decode.batch == 3 && g_decode_sq == S && g_decode.num_parts == P && g_decode_fp8 == fp8,
                 "decode parameters B=%d S=%d P=%d", g_decode.batch, g_decode_sq, g_decode.num_parts);
          EXPECT(g_decode.max_blocks == 8, "max_blocks %d", g_decode.max_blocks);
          EXPECT((g_decode.block_table != nullptr) == paged, "block table pointer");
          EXPECT((g_decode.part_lse != nullptr) == (P > 1), "partials passed only when split");
          EXPECT(std::fabs(g_decode.scale_log2 - c.scale * 1.4426950408889634f) < 1e-7f, "scale_log2");
        }
  // each argument broken in turn
  struct Case {
    const char* what;
    mla_status want;
    void (*edit)(DecodeCall&);
  };
  const Case cases[] = {
      {"q dtype", MLA_ERR_DTYPE, [](DecodeCall& c) { c.q.dtype = MLA_DTYPE_FP32; }},
      {"q heads 64", MLA_ERR_SHAPE, [](DecodeCall& c) { c.q = dense(MLA_DTYPE_BF16, {3, 2, 64, 512}); }},
      {"q width 576", MLA_ERR_SHAPE, [](DecodeCall& c) { c.q = dense(MLA_DTYPE_BF16, {3, 2, 128, 576}); }},
      {"q rank 3", MLA_ERR_SHAPE, [](DecodeCall& c) { c.q = dense(MLA_DTYPE_BF16, {6, 128, 512}); }},
      {"q strided", MLA_ERR_SHAPE, [](DecodeCall& c) { c.q.strides[2] = 1024; }},
      {"q null", MLA_ERR_NULL, [](DecodeCall& c) { c.q.data = nullptr; }},
      {"q_rope width", MLA_ERR_SHAPE, [](DecodeCall& c) { c.qr = dense(MLA_DTYPE_BF16, {3, 2, 128, 32}); }},
      {"lens batch", MLA_ERR_SHAPE, [](DecodeCall& c) { c.lens = dense(MLA_DTYPE_INT32, {4}); }},
      {"lens dtype", MLA_ERR_DTYPE, [](DecodeCall& c) { c.lens.dtype = MLA_DTYPE_FP32; }},
      {"out null", MLA_ERR_NULL, [](DecodeCall& c) { c.out.data = nullptr; }},
      {"out dtype", MLA_ERR_DTYPE, [](DecodeCall& c) { c.out.dtype = MLA_DTYPE_BF16; }},
      {"lse batch", MLA_ERR_SHAPE, [](DecodeCall& c) { c.lse = dense(MLA_DTYPE_FP32, {4, 2, 128}); }},
      {"65 tokens", MLA_ERR_UNSUPPORTED, [](DecodeCall& c) {
         c.out = dense(MLA_DTYPE_FP32, {3, 65, 128, 512});
         c.lse = dense(MLA_DTYPE_FP32, {3, 65, 128});
       }},
      {"table batch", MLA_ERR_SHAPE, [](DecodeCall& c) { c.table = dense(MLA_DTYPE_INT32, {2, 8}); }},
      {"table dtype", MLA_ERR_DTYPE, [](DecodeCall& c) { c.table.dtype = MLA_DTYPE_UINT8; }},
      {"cache width", MLA_ERR_SHAPE, [](DecodeCall& c) { c.cache.rows = dense(MLA_DTYPE_BF16, {40, 64, 512}); }},
      {"cache pages of 32", MLA_ERR_UNSUPPORTED,
       [](DecodeCall& c) { c.cache.rows = dense(MLA_DTYPE_BF16, {40, 32, 576}); }},
      {"cache pages of 48", MLA_ERR_SHAPE, [](DecodeCall& c) { c.cache.rows = dense(MLA_DTYPE_BF16, {40, 48, 576}); }},
      {"cache dtype", MLA_ERR_DTYPE, [](DecodeCall& c) { c.cache.rows.dtype = MLA_DTYPE_FP32; }},
      {"scale NaN", MLA_ERR_SHAPE, [](DecodeCall& c) { c.scale = std::nanf(""); }},
      {"splits 3", MLA_ERR_SHAPE, [](DecodeCall& c) { c.plse = dense(MLA_DTYPE_FP32, {3, 2, 2, 128}); }},
      {"splits too many", MLA_ERR_SHAPE,
       [](DecodeCall& c) { c.plse = dense(MLA_DTYPE_FP32, {2 * (int64_t)MLA_MAX_SPLITS, 2, 2, 128}); }},
      {"partial_out short", MLA_ERR_SHAPE, [](DecodeCall& c) { c.pout.shape[0] -= 1; }},
      {"partial_out misaligned", MLA_ERR_SHAPE,
       [](DecodeCall& c) { c.pout.data = static_cast<char*>(c.pout.data) + 8; }},
      {"partial_out missing", MLA_ERR_NULL, [](DecodeCall& c) { c.pout.data = nullptr; }},
      {"q misaligned", MLA_ERR_SHAPE, [](DecodeCall& c) { c.q.data = static_cast<char*>(c.q.data) + 4; }},
      {"cache rows misaligned", MLA_ERR_SHAPE,
       [](DecodeCall& c) { c.cache.rows.data = static_cast<char*>(c.cache.rows.data) + 8; }},
      {"lengths misaligned", MLA_ERR_SHAPE,
       [](DecodeCall& c) { c.lens.data = static_cast<char*>(c.lens.data) + 2; }},
      {"out misaligned", MLA_ERR_SHAPE, [](DecodeCall& c) { c.out.data = static_cast<char*>(c.out.data) + 4; }},
      {"sizes past any memory", MLA_ERR_SHAPE, [](DecodeCall& c) {
         c.table = dense(MLA_DTYPE_INT32, {3, (int64_t)1 << 50});
       }},
  };
  for (const Case& k : cases) {
    DecodeCall c(3, 2, 4, false, true);
    k.edit(c);
    const int before = g_decode_launches;
    const mla_status st = c.run();
    EXPECT(st == k.want, "decode with %s: status %d, expected %d", k.what, st, k.want);
    EXPECT(g_decode_launches == before, "decode with %s launched", k.what);
  }
  // e4m3 bundle
  {
    DecodeCall c(2, 1, 1, true, true);
    c.cache.scales.data = nullptr;
    EXPECT(c.run() == MLA_ERR_NULL, "e4m3 without scales");
    DecodeCall d(2, 1, 1, true, true);
    d.cache.rope = dense(MLA_DTYPE_BF16, {40, 64, 32});
    EXPECT(d.run() == MLA_ERR_SHAPE, "e4m3 rope width");
    DecodeCall e(2, 1, 1, true, true);
    e.cache.scales = dense(MLA_DTYPE_FP32, {41, 64, 4});
    EXPECT(e.run() == MLA_ERR_SHAPE, "e4m3 scales pages");
  }
  // contiguous cache shapes: [B * max_blocks, 64, .] or [B, L_cap, .]
  {
    DecodeCall c(3, 1, 1, false, false);
    c.cache.rows = dense(MLA_DTYPE_BF16, {3, 256, 576});
    EXPECT(c.run() == MLA_OK && g_decode.max_blocks == 4, "contiguous [B, L_cap, 576]");
    DecodeCall d(3, 1, 1, false, false);
    d.cache.rows = dense(MLA_DTYPE_BF16, {4, 256, 576});
    EXPECT(d.run() == MLA_ERR_SHAPE, "contiguous cache of another batch");
  }
}

void directed_others() {
  // combine: partials of a decode, and no launch without partials
  {
    DecodeCall c(5, 2, 8, false, true);
    const int before = g_combine_launches;
    EXPECT(mla_combine(&c.pout, &c.plse, &c.lens, &c.out, &c.lse, nullptr) == MLA_OK, "combine");
    EXPECT(g_combine_launches == before + 1 && g_combine.num_parts == 8 && g_combine.log2_parts == 3 &&
               g_combine.batch == 5 && g_combine.s_q == 2,
           "combine parameters");
    EXPECT(mla_combine(nullptr, nullptr, &c.lens, &c.out, &c.lse, nullptr) == MLA_OK &&
               g_combine_launches == before + 1,
           "combine without partials launches nothing");
  }
  // no-alloc decode: split bound and the scratch
  {
    DecodeCall c(2, 2, 1, false, true);
    const mla_status ok = mla_decode_noalloc(&c.q, &c.qr, &c.cache, &c.table, &c.lens, c.scale, &c.out, &c.lse,
                                             128, nullptr);
    EXPECT(ok == MLA_OK && g_decode.num_parts == 128 && g_decode.part_out != nullptr, "noalloc 128 x 2");
    EXPECT(mla_decode_noalloc(&c.q, &c.qr, &c.cache, &c.table, &c.lens, c.scale, &c.out, &c.lse, 256, nullptr) ==
               MLA_ERR_SCRATCH,
           "noalloc 256 x 2 over the scratch");
    EXPECT(mla_decode_noalloc(&c.q, &c.qr, &c.cache, &c.table, &c.lens, c.scale, &c.out, &c.lse, 6, nullptr) ==
               MLA_ERR_SHAPE,
           "noalloc split count not a power of two");
  }
  // the projections
  {
    mla_tensor qc = dense(MLA_DTYPE_BF16, {4, 2, 128, 128}), qr = dense(MLA_DTYPE_BF16, {4, 2, 128, 64});
    mla_tensor w = dense(MLA_DTYPE_BF16, {128, 512, 128}), lens = dense(MLA_DTYPE_INT32, {4});
    mla_tensor qa = dense(MLA_DTYPE_BF16, {4, 2, 128, 512}), qro = dense(MLA_DTYPE_BF16, {4, 2, 128, 64});
    EXPECT(mla_absorb_query(&qc, &qr, &w, &lens, 10000.f, &qa, &qro, nullptr) == MLA_OK, "absorb_query");
    EXPECT(mla_absorb_query(&qc, &qr, &w, &lens, -1.f, &qa, &qro, nullptr) == MLA_ERR_SHAPE, "rope base");
    mla_tensor wt = dense(MLA_DTYPE_BF16, {128, 128, 512});
    EXPECT(mla_absorb_query(&qc, &qr, &wt, &lens, 10000.f, &qa, &qro, nullptr) == MLA_ERR_SHAPE,
           "W^UK not transposed");
    mla_tensor ol = dense(MLA_DTYPE_FP32, {4, 2, 128, 512}), wv = dense(MLA_DTYPE_BF16, {128, 128, 512});
    mla_tensor ov = dense(MLA_DTYPE_FP32, {4, 2, 128, 128});
    EXPECT(mla_absorb_output(&ol, &wv, &ov, nullptr) == MLA_OK, "absorb_output");
    ov.data = static_cast<char*>(ov.data) + 4;
    EXPECT(mla_absorb_output(&ol, &wv, &ov, nullptr) == MLA_ERR_SHAPE, "absorb_output misaligned");
    mla_tensor h = dense(MLA_DTYPE_BF16, {70, 7168}), wk = dense(MLA_DTYPE_BF16, {576, 7168});
    mla_tensor kv = dense(MLA_DTYPE_FP32, {70, 576});
    EXPECT(mla_kv_project(&h, &wk, &kv, nullptr) == MLA_OK, "kv_project");
    mla_tensor h2 = dense(MLA_DTYPE_BF16, {70, 7072}), wk2 = dense(MLA_DTYPE_BF16, {576, 7072});
    EXPECT(mla_kv_project(&h2, &wk2, &kv, nullptr) == MLA_ERR_SHAPE, "hidden size not a multiple of 128");
    mla_tensor kws = dense(MLA_DTYPE_FP32, {28, 70, 576}), kws5 = dense(MLA_DTYPE_FP32, {5, 70, 576});
    EXPECT(mla_kv_project_split(&h, &wk, &kv, &kws, nullptr) == MLA_OK, "kv_project_split");
    EXPECT(mla_kv_project_split(&h, &wk, &kv, &kws5, nullptr) == MLA_ERR_SHAPE, "slices not dividing d / 128");
    EXPECT(mla_kv_project_split(&h, &wk, &kv, nullptr, nullptr) == MLA_ERR_NULL, "no workspace");
    EXPECT(mla_kv_project_splits(70, 7168) == 28 && mla_kv_project_splits(1, 100) == 0, "split hint");
    mla_tensor kv3 = dense(MLA_DTYPE_FP32, {4, 2, 576});
    DecodeCall c(4, 2, 1, true, true);
    EXPECT(mla_cache_append(&kv3, &c.lens, &c.table, &c.cache, 10000.f, nullptr) == MLA_OK, "cache append");
    mla_tensor counts = dense(MLA_DTYPE_INT32, {2});
    EXPECT(mla_check_indices(&c.cache, &c.table, &c.lens, &counts, nullptr) == MLA_OK, "check_indices");
    mla_tensor counts3 = dense(MLA_DTYPE_INT32, {3});
    EXPECT(mla_check_indices(&c.cache, &c.table, &c.lens, &counts3, nullptr) == MLA_ERR_SHAPE, "counts [3]");
  }
  EXPECT(mla_init(0) == MLA_OK, "init on the gfx950 stub");
  EXPECT(mla_init(1) == MLA_ERR_DEVICE, "init on a missing device");
  EXPECT(mla_num_splits_hint(0, 128, 2, 128) == 128, "hint for 128 x 2 tokens: %d", mla_num_splits_hint(0, 128, 2, 128));
  EXPECT(mla_num_splits_hint(0, 1, 1, 2) == 1, "hint for one short sequence");
  EXPECT(mla_num_splits_hint(0, 0, 1, 2) == 0 && mla_num_splits_hint(0, 4, 65, 2) == 0, "hint refusals");
  EXPECT(mla_partial_out_bytes(0, 1) == 0 && mla_partial_out_bytes(4, 0) == 0, "workspace sizes of nothing");
  for (int s = 0; s <= 8; ++s) EXPECT(mla_status_string((mla_status)s) != nullptr, "status text %d", s);
  EXPECT(mla_status_string((mla_status)1234) != nullptr, "text of an unknown status");
}

// any bits in a descriptor: a status comes back, nothing launches
void random_tensor(std::mt19937_64& g, mla_tensor* t) {
  const int64_t pick[] = {-1, 0, 1, 2, 3, 4, 5, 64, 128, 512, 576, 7168, (int64_t)1 << 31, (int64_t)1 << 62,
                          INT64_MIN, INT64_MAX};
  auto any = [&]() { return (g() & 1) ? pick[g() % 16] : (int64_t)(g() % 1000) - 10; };
  t->data = (g() % 8) ? reinterpret_cast<void*>(uintptr_t(g() & ~uint64_t(0xf)) | 0x1000) : nullptr;
  t->dtype = (int32_t)((g() % 4) ? g() % 6 : g());
  t->rank = (int32_t)((g() % 4) ? g() % 7 : g());
  for (int k = 0; k < 5; ++k) {
    t->shape[k] = any();
    t->strides[k] = (g() % 3) ? 0 : any();
  }
  if (g() % 2) {  // dense strides, so that more cases reach the later checks
    int64_t s = 1;
    for (int k = 4; k >= 0; --k) {
      t->strides[k] = s;
      if (t->shape[k] > 0 && t->shape[k] < (int64_t)1 << 20) s *= t->shape[k];
    }
  }
}

void fuzz(int iters) {
  std::mt19937_64 g(12345);
  const int launches = g_decode_launches + g_combine_launches + g_gemm_launches + g_other_launches;
  int ok = 0;
  for (int i = 0; i < iters; ++i) {
    mla_tensor t[9];
    for (auto& x : t) random_tensor(g, &x);
    mla_latent_cache c{};
    random_tensor(g, &c.rows);
    random_tensor(g, &c.scales);
    random_tensor(g, &c.rope);
    auto maybe = [&](mla_tensor* x) { return (g() % 6) ? x : nullptr; };
    const float f = (g() % 5) ? 0.07f : ((g() % 2) ? std::nanf("") : -3.f);
    mla_status st;
    switch (g() % 9) {
      case 0: st = mla_decode(maybe(&t[0]), maybe(&t[1]), (g() % 6) ? &c : nullptr, maybe(&t[2]), maybe(&t[3]), f,
                              maybe(&t[4]), maybe(&t[5]), maybe(&t[6]), maybe(&t[7]), nullptr); break;
      case 1: st = mla_combine(maybe(&t[0]), maybe(&t[1]), maybe(&t[2]), maybe(&t[3]), maybe(&t[4]), nullptr); break;
      case 2: st = mla_decode_noalloc(maybe(&t[0]), maybe(&t[1]), (g() % 6) ? &c : nullptr, maybe(&t[2]),
                                      maybe(&t[3]), f, maybe(&t[4]), maybe(&t[5]), (int32_t)g(), nullptr); break;
      case 3: st = mla_absorb_query(maybe(&t[0]), maybe(&t[1]), maybe(&t[2]), maybe(&t[3]), f, maybe(&t[4]),
                                    maybe(&t[5]), nullptr); break;
      case 4: st = mla_absorb_output(maybe(&t[0]), maybe(&t[1]), maybe(&t[2]), nullptr); break;
      case 5: st = (g() % 2) ? mla_kv_project(maybe(&t[0]), maybe(&t[1]), maybe(&t[2]), nullptr)
                             : mla_kv_project_split(maybe(&t[0]), maybe(&t[1]), maybe(&t[2]), maybe(&t[3]), nullptr);
              break;
      case 6: st = mla_cache_append(maybe(&t[0]), maybe(&t[1]), maybe(&t[2]), (g() % 6) ? &c : nullptr, f, nullptr); break;
      case 7: st = mla_check_indices((g() % 6) ? &c : nullptr, maybe(&t[0]), maybe(&t[1]), maybe(&t[2]), nullptr); break;
      default: (void)mla_num_splits_hint((int32_t)(g() % 3), (int32_t)g(), (int32_t)g(), (int32_t)g());
               (void)mla_partial_out_bytes((int32_t)g(), (int32_t)g());
               (void)mla_partial_lse_bytes((int32_t)g(), (int32_t)g());
               st = MLA_ERR_SHAPE;
    }
    EXPECT((int)st >= 0 && (int)st <= 7, "fuzz case %d: status %d", i, (int)st);
    ok += st == MLA_OK;
  }
  (void)launches;
  std::printf("fuzz: %d random calls, %d accepted\n", iters, ok);
}
// valid decode calls with one or two fields changed to arbitrary values: an
// accepted call launches once, with parameters that match its descriptors
void mutate(int iters) {
  std::mt19937_64 g(777);
  const int64_t pick[] = {-7, -1, 0, 1, 2, 3, 4, 8, 63, 64, 65, 128, 512, 576, 1 << 20, (int64_t)1 << 40,
                          INT64_MAX, INT64_MIN};
  int accepted = 0;
  for (int i = 0; i < iters; ++i) {
    const int64_t B = 1 + (int64_t)(g() % 6), S = 1 + (int64_t)(g() % 5), P = (int64_t)1 << (g() % 5);
    DecodeCall c(B, S, P, g() % 2, g() % 2);
    mla_tensor* fields[] = {&c.q, &c.qr, &c.table, &c.lens, &c.out, &c.lse, &c.pout, &c.plse,
                            &c.cache.rows, &c.cache.scales, &c.cache.rope};
    for (int m = 0, n = 1 + (int)(g() % 2); m < n; ++m) {
      mla_tensor* f = fields[g() % 11];
      switch (g() % 5) {
        case 0: f->shape[g() % 5] = pick[g() % 18]; break;
        case 1: f->strides[g() % 5] = pick[g() % 18]; break;
        case 2: f->rank = (int32_t)(g() % 7); break;
        case 3: f->dtype = (int32_t)(g() % 6); break;
        default:
          if (g() % 2 || f->data == nullptr) f->data = nullptr;
          else f->data = static_cast<char*>(f->data) + 4 * (g() % 4);
      }
    }
    const int before = g_decode_launches;
    const mla_status st = c.run();
    EXPECT((int)st >= 0 && (int)st <= 7, "mutation %d: status %d", i, (int)st);
    if (st == MLA_OK) {
      ++accepted;
      EXPECT(g_decode_launches == before + 1, "mutation %d: accepted without one launch", i);
      EXPECT(g_decode.batch == c.out.shape[0] && g_decode_sq == c.out.shape[1], "mutation %d: B, S", i);
      EXPECT(g_decode.num_parts >= 1 && (g_decode.num_parts & (g_decode.num_parts - 1)) == 0,
             "mutation %d: split count %d", i, g_decode.num_parts);
      EXPECT(g_decode.max_blocks >= 1, "mutation %d: max_blocks %d", i, g_decode.max_blocks);
      EXPECT(((uintptr_t)g_decode.q_abs & 15) == 0 && ((uintptr_t)g_decode.rows & 15) == 0 &&
                 ((uintptr_t)g_decode.out & 15) == 0 && ((uintptr_t)g_decode.seq_lens & 3) == 0,
             "mutation %d: misaligned pointer accepted", i);
    } else {
      EXPECT(g_decode_launches == before, "mutation %d: refused (%d) yet launched", i, (int)st);
    }
  }
  std::printf("mutations: %d changed valid calls, %d still accepted\n", iters, accepted);
}
}  // namespace

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 200000;
  directed_decode();
  directed_others();
  fuzz(iters);
  mutate(iters / 4);
  if (g_fail) {
    std::printf("%d check(s) failed\n", g_fail);
    return 1;
  }
  std::printf("OK\n");
  return 0;
}
