// The scratch memory of wushkv_decode_step_noalloc: a file-scope device array
// that holds the decode workspace (split partials and per-unit query blocks)
// for callers that cannot allocate.  Each GPU holds its own copy for the life
// of the process; its device address is looked up once per device and kept.
#include <mutex>

#include "common.h"

namespace wkv {

constexpr uint64_t NOALLOC_SCRATCH_BYTES = WUSHKV_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_ptr[MAX_DEVICES];  // device address of `scratch` per device (null until looked up)
}  // namespace

// Device address and size of the current device's scratch array.  The array's
// name is only a host-side stand-in, so every use of the memory (kernel
// arguments) goes through this address.
hipError_t noalloc_scratch(void** ptr, uint64_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  *bytes = NOALLOC_SCRATCH_BYTES;
  return hipSuccess;
}

}  // namespace wkv
