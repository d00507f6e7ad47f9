// Device scratch for the entry point that allocates nothing
// (tpc_conv_fwd_noalloc): a fixed file-scope array in device memory, one copy
// per GPU, held until the process ends.  Host code never uses the array's
// name as an address (on the host it only stands for the symbol): the device
// address of each GPU's copy is looked up once per device with
// hipGetSymbolAddress, with that device current, and cached here.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.hpp"

namespace tpc {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t scratch_for_current_device(void** ptr, size_t* bytes) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  *bytes = kNoAllocScratchBytes;
  return hipSuccess;
}

}  // namespace tpc
