// Library-owned scratch memory for the entry point that allocates nothing
// (fa_backward_noalloc): the backward preprocess's two float32 per query row
// (D = rowsum(dO * O) and LSE * log2 e) live in one file-scope device array
// instead of a caller-provided workspace.
//
// The array exists once per device the library runs on, for the life of the
// process.  Its device address is looked up with hipGetSymbolAddress, once
// per device with that device current, and kept; host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the
// symbol).  Every call on one device shares that device's array, so calls
// that overlap on one device (e.g. on two streams) race; the backward's
// preprocess writes every row of it before the other kernels read it, so
// nothing needs clearing between calls.
#include <mutex>

#include "fa_kernels.h"

namespace fa {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device once looked up
}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, void** ptr) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace fa
