// fa_static.hip -- the library's one static device buffer, used by the
// backward entry point that allocates nothing (fa_bwd_static, include/fa.h).
//
// `scratch` holds the backward's row term D (4 bytes per query row) in place
// of a caller-provided workspace.  Every GPU the library runs on holds its
// own copy from the module load until the process ends.  In host code the
// array's name is only a host-side handle: its device address is looked up
// once per device with hipGetSymbolAddress (with that device current) and
// kept, and only that address is ever handed to kernels.

#include <mutex>

#include "../../include/fa.h"
#include "fa_launch.hpp"

namespace fa {

static __device__ __align__(256) unsigned char scratch[FA_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_lookup;
void* g_addr[kMaxDevices];      // device address of `scratch`, per device
}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_lookup);
  if (!g_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_addr[dev] = p;
  }
  *ptr = g_addr[dev];
  return hipSuccess;
}

}  // namespace fa
