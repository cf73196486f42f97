// Device scratch of the no-allocation entry point (mla_decode_noalloc): one
// file-scope array per GPU, so that a caller that cannot allocate (code under
// graph capture, allocation-free serving loops) still gets the decode's
// workspace.  Its host-side name is only a stand-in for the symbol: the
// device address of each GPU's copy comes from hipGetSymbolAddress, taken
// once per device with that device current, and only that address is ever
// passed to kernels or copies.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mla_common.h"

namespace mla {

static __device__ __align__(256) char scratch[kScratchBytes];

hipError_t scratch_address(void** out) {
  constexpr int kMaxDevices = 64;
  static std::once_flag once[kMaxDevices];
  static void* addr[kMaxDevices];
  static hipError_t err[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(once[dev], [dev] {
    void* p = nullptr;
    err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    addr[dev] = p;
  });
  if (err[dev] != hipSuccess) return err[dev];
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace mla
