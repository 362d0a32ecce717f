// fa_scratch.hip -- the library's own device scratch buffer, for the gradient entry point that allocates nothing
// (fa_bwd_noalloc): a file-scope device array of kScratchBytes, one copy on every GPU the library runs on, held
// until the process ends. Host code never passes the array's name to a kernel (in host code it is only a stand-in
// for the symbol); it looks the array's device address up once per device, with that device current, and hands
// that address to the kernels as their workspace.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "fa_launch.h"

static __device__ __align__(256) unsigned char scratch[fa::kScratchBytes];

namespace fa {

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_addr[kMaxDevices];  // device address of `scratch` per device, once looked up
std::mutex g_lookup;
}  // namespace

hipError_t scratch_address(hipStream_t stream, void** out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (stream) {  // the device the stream belongs to (the null stream is the current device's)
    hipDevice_t sd = 0;
    e = hipStreamGetDevice(stream, &sd);
    if (e != hipSuccess) return e;
    dev = sd;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_lookup);
    p = g_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (dev != cur) {
        const hipError_t e2 = hipSetDevice(cur);
        if (e == hipSuccess) e = e2;
      }
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace fa
