// Device-resident scratch for the entry point that allocates nothing (mla_decode_noalloc):
// the split partials of the attention live in a fixed file-scope device array instead of a
// caller workspace.  Every GPU the library runs on holds its own copy of the array until the
// process ends; the host finds that copy's address once per device with
// hipGetSymbolAddress (the array's name is only a host-side stand-in, never a device
// address) and uses that pointer from then on.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launchers.h"

namespace mla {
namespace {

constexpr size_t kScratchBytes = size_t{48} << 20;  // 48 MiB of split partials
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

void* g_scratch[kMaxDevices] = {};
std::mutex g_scratch_mu;

}  // namespace

size_t noalloc_scratch_bytes() { return kScratchBytes; }

hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // this device's copy, it being current
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace mla
