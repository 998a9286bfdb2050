// The workspace of tri_attn_forward_noalloc: a static device array, one copy
// per GPU, so that callers that must not allocate (code under graph capture,
// tight serving loops, harnesses that forbid allocation) can run the forward
// without a workspace argument. Each GPU the library runs on holds its copy
// until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "tri_attn.h"
#include "tri_attn_internal.h"

namespace tpa {

static __device__ __align__(256) unsigned char scratch[TRI_ATTN_NOALLOC_MAX_BYTES];

constexpr int kMaxDevices = 64;

// The device address of this GPU's copy of `scratch`, looked up with
// hipGetSymbolAddress once per device (the caller makes `device` current).
// In host code the array's name is only a host-side stand-in: nothing but
// the address returned here may reach a kernel or a runtime call.
int scratch_address(int device, void **ptr) {
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  *ptr = nullptr;
  if (device < 0 || device >= kMaxDevices) return TRI_ATTN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[device]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return TRI_ATTN_ERR_HIP;
    }
    addr[device] = p;
  }
  *ptr = addr[device];
  return TRI_ATTN_OK;
}

}  // namespace tpa
