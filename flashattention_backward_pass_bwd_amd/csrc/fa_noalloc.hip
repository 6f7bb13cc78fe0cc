// The library-owned dS workspace of fa_bwd_dkdv_dq_noalloc, for callers that
// cannot allocate device memory (HIP graph capture, serving loops, harnesses
// that forbid hipMalloc).
//
// `scratch` is a file-scope device array: every GPU the library runs on holds
// its own copy, at its own address, from the first launch on that device until
// the process ends.  In host code the name `scratch` only stands for the
// symbol; its device address is fetched once per device with
// hipGetSymbolAddress (with that device current) and cached here, and only
// that address is ever handed to a kernel.  Calls on one GPU share its copy:
// calls that overlap on one GPU (different streams, no ordering) race.
#include <mutex>

#include "fa_bwd.h"
#include "fa_internal.h"

static __device__ __align__(256) unsigned char scratch[FA_BWD_NOALLOC_SCRATCH_BYTES];

namespace fa {

namespace {
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device id, once fetched
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace fa
