// The scratch array behind velox_route_noalloc: a file-scope device array of
// VELOX_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds until
// the process ends.  In host code the array's name is only a stand-in for the
// symbol, not a device address: its address on a device comes from
// hipGetSymbolAddress with that device current, looked up once per device
// and kept.
#include <mutex>

#include "velox_internal.h"

namespace velox {
namespace {

static __device__ __align__(256) unsigned char scratch[VELOX_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t device_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace velox
