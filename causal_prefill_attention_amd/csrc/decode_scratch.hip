// Static device scratch of the decode split for callers that cannot
// allocate (attn_decode_noalloc): code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "prefill_params.h"

namespace attnp {

// Split partials of attn_decode_noalloc, for callers that cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): kDecodeScratchBytes of device memory that every GPU the
// library runs on holds until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the
// symbol); it uses the address decode_static_scratch looks up per device.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_static_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    // once per device, with that device current: each GPU holds its own
    // copy of the array at its own address
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace attnp
