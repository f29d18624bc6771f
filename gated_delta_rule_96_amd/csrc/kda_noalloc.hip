// Allocation-free chunked prefill: the fused schedule of kda_fwd_chunked
// with its ring buffers and control words in a library-owned device array
// instead of a caller-supplied workspace, for callers that cannot allocate
// (code under graph capture, serving loops, harnesses that forbid it).
//
// `scratch` is a file-scope device array: one copy per GPU, created when
// the code object is loaded there and held until the process ends.  In host
// code its name is a host-side stand-in, not a device address, so it is
// never passed to a kernel; the device address comes from
// hipGetSymbolAddress, fetched once per device (with that device current)
// on the first call there and kept.  Every call on one GPU shares that
// GPU's array: calls that overlap on one GPU (different streams, no
// ordering between them) race on it.  Its flags and status word are
// cleared by kernels on the caller's stream at the start of each call.
#include <mutex>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace kda
