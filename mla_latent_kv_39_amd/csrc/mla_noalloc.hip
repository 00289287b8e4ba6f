// Static scratch of mla_decode_noalloc: the split partials (fp16 partial_out
// blocks with their descales, then partial_lse) of one decode + combine live
// in a file-scope device array instead of a caller's workspace, so that a
// caller that cannot allocate (graph capture, a serving loop) still gets the
// split-KV decode.  Each device that loads the library holds its own copy of
// the array until the process ends; its address is taken once per device
// (mla_init, else the first mla_decode_noalloc on the device) and kept.
#include <mutex>

#include "mla_internal.h"

namespace mla {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    // the array's device address on the current device; the name itself is a
    // host-side stand-in and is never passed to a kernel
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace mla
