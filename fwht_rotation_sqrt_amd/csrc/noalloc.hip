// The library's one static device buffer, for the entry point that allocates
// nothing (tb_linear_noalloc): x' of a batched linear lives here instead of in a
// caller workspace.  Every GPU the library runs on holds its own copy of the
// array until the process ends.  Host code never uses the array's name as an
// address (on the host it is only a stand-in for the symbol): the device
// address comes from hipGetSymbolAddress, once per device, with that device
// current, and is kept per device.
#include "tb_internal.hpp"

#include <mutex>

namespace tb {
namespace {

static __device__ __align__(256) float scratch[kStaticScratchFloats];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
  });
  *ptr = g_ptr[dev];
  return g_err[dev];
}

}  // namespace tb
