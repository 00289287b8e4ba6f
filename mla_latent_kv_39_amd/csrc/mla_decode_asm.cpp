// Host launcher of the assembly decode kernels (bf16 and fp8 cache), generated
// by gen_decode_gfx950.py and assembled into one code object that is embedded
// in libmla.so and loaded once per device (by mla_init or on first use).
#include <mutex>

#include "mla_internal.h"

extern "C" const unsigned char mla_decode_gfx950_co[];
extern "C" const unsigned long mla_decode_gfx950_co_size;

namespace mla {
namespace {

// Kernel argument block; layout fixed by the kernel's s_load offsets.
struct AsmArgs {
  const void* q_abs;
  const void* q_rope;
  const void* rows;
  const void* table;
  const int32_t* seq_lens;
  void* part_out;
  float* part_lse;
  float* out;
  float* lse;
  float scale_log2;
  int32_t max_blocks;
  int32_t batch;
  int32_t num_parts;
  int32_t s_q;
  int32_t heads_per_block;
  int32_t head_blocks;
  int32_t log2_parts;
  const float* fp8_scales;  // fp8 cache only
  const void* fp8_rope;     // fp8 cache only
  int32_t tok_stride;       // query tokens per sequence in q, out, lse and the partials
  int32_t tok0;             // the first token of this launch's group
};
static_assert(sizeof(AsmArgs) == 128, "kernel argument layout");

constexpr int kMaxDevices = 64;
std::mutex g_mu;
hipModule_t g_mod[kMaxDevices];
hipFunction_t g_fn[kMaxDevices][2];   // [bf16, fp8]

hipError_t decode_function(bool fp8, hipFunction_t* fn) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  // the code object is loaded once per device and kept until the process ends
  if (!g_mod[dev]) {
    hipModule_t mod;
    err = hipModuleLoadData(&mod, mla_decode_gfx950_co);
    if (err != hipSuccess) return err;
    err = hipModuleGetFunction(&g_fn[dev][0], mod, "mla_decode_bf16_gfx950");
    if (err == hipSuccess) err = hipModuleGetFunction(&g_fn[dev][1], mod, "mla_decode_fp8_gfx950");
    if (err != hipSuccess) {
      hipModuleUnload(mod);
      return err;
    }
    g_mod[dev] = mod;
  }
  *fn = g_fn[dev][fp8 ? 1 : 0];
  return hipSuccess;
}

}  // namespace

hipError_t load_decode_module() {
  hipFunction_t fn;
  return decode_function(false, &fn);
}

hipError_t launch_decode(const DecodeParams& p, int s_q, bool fp8, hipStream_t stream) {
  hipFunction_t fn;
  hipError_t err = decode_function(fp8, &fn);
  if (err != hipSuccess) return err;
  int lg = 0;
  while ((1 << lg) < p.num_parts) ++lg;
  // a workgroup holds 128 query rows, four waves of 32 heads of one token: the
  // tokens go out in groups of 4, 2 and 1, each group one launch over the same
  // partitions (the partition map depends on the lengths only)
  for (int tok0 = 0; tok0 < s_q;) {
    const int group = token_group(s_q - tok0);
    AsmArgs a;
    a.q_abs = p.q_abs;
    a.q_rope = p.q_rope;
    a.rows = p.rows;
    a.table = p.block_table;
    a.seq_lens = p.seq_lens;
    a.part_out = p.part_out;
    a.part_lse = p.part_lse;
    a.out = p.out;
    a.lse = p.lse;
    a.scale_log2 = p.scale_log2;
    a.max_blocks = p.max_blocks;
    a.batch = p.batch;
    a.num_parts = p.num_parts;
    a.s_q = group;
    a.heads_per_block = heads_per_block(group);
    a.head_blocks = kHeads / a.heads_per_block;
    a.log2_parts = lg;
    a.fp8_scales = p.fp8_scales;
    a.fp8_rope = p.fp8_rope;
    a.tok_stride = s_q;
    a.tok0 = tok0;
    size_t size = sizeof(a);
    void* config[] = {HIP_LAUNCH_PARAM_BUFFER_POINTER, &a, HIP_LAUNCH_PARAM_BUFFER_SIZE, &size,
                      HIP_LAUNCH_PARAM_END};
    err = hipModuleLaunchKernel(fn, (unsigned)(p.num_parts * a.head_blocks), 1, 1, 256, 1, 1, 0, stream, nullptr,
                                config);
    if (err != hipSuccess) return err;
    tok0 += group;
  }
  return hipSuccess;
}

}  // namespace mla
