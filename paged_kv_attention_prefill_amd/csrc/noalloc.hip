// Library-owned scratch memory for the entry point that allocates nothing
// (paged_attn_decode_noalloc): the workspace of a decode call (partial states
// of internal KV splits and the balanced split's per-item workgroup spans) is
// taken from a file-scope device array instead of a caller buffer.
//
// `scratch` names a host-side stand-in in host code, not a device address: its
// device address is read once per device with hipGetSymbolAddress (with that
// device current) and kept per device; every GPU holds its own copy of the
// array, allocated when the code object loads and held until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "params.h"

namespace pa {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDev = 64;
std::once_flag g_once[kMaxDev];
void* g_ptr[kMaxDev];
hipError_t g_err[kMaxDev];

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_err[dev] != hipSuccess) return g_err[dev];
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace pa
