// Scratch of the allocation-free attention entry point: one static device
// array per GPU for the key-range split partials.
//
// It lives in a source file of its own, so it is a code object of its own:
// the runtime loads a code object, and sets up its device globals, on the
// first use of anything in it.  In the attention kernel's file the array
// would make every process pay for a 128 MiB device global at its first
// attention launch (~50 ms, measured); here only the first lookup below
// pays, once per device.
//
// Host code never passes the array's name to a kernel (on the host it is
// only a stand-in, not a device address): it passes the address that
// scratch_region() looked up with hipGetSymbolAddress for the current device.
#include "../wm_internal.hpp"

#include <mutex>

namespace wm {

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch[kMaxDevices];
}  // namespace

hipError_t scratch_region(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

}  // namespace wm
