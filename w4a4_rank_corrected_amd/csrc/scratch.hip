// Device-resident scratch memory of the allocation-free entry point
// (svdq_linear_noalloc): a file-scope device array of kScratchBytes that each
// GPU the library runs on holds until the process ends.  Host code never
// passes the array's name to a kernel (on the host it only stands for the
// symbol): its device address is looked up once per device with
// hipGetSymbolAddress and cached, and that address is what the kernels get.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace svdq {
namespace {

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

}  // namespace

int scratch_buffer(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with `dev` current
    if (e != hipSuccess) return (int)e;
    if (p == nullptr || ((uintptr_t)p & 255u) != 0) return (int)hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return 0;
}

}  // namespace svdq
