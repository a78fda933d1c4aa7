// Device scratch for mla_decode_latent_noalloc: a file-scope device array
// that holds the split-KV partials, so that call allocates nothing.
//
// Each GPU the library runs on holds its own copy of the array (kScratchBytes)
// until the process ends.  Host code never uses the array's name as a device
// address: the address comes from hipGetSymbolAddress, looked up once per
// device with that device current, and is kept per device.  Every call on a
// GPU shares that GPU's array, so calls that overlap on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.hpp"

namespace mla {

namespace {

static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t scratch_region(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace mla
