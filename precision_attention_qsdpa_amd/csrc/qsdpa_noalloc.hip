// qsdpa_forward without a caller workspace and without any allocation: the
// workspace (codes, scales, statistics partials and, in FP4 mode, the
// expanded K) lives in one file-scope device array, `scratch`, of
// QSDPA_SCRATCH_BYTES.  Each GPU the library runs on holds its own copy of
// the array until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device with hipGetSymbolAddress (with
// that device current) and only that address is ever passed to kernels.
#include <hip/hip_runtime.h>

#include <atomic>

#include "../../include/qsdpa.h"
#include "qsdpa_launch.h"

namespace {

static __device__ __align__(256) uint8_t scratch[QSDPA_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_ptr[kMaxDevices];

// Device address of this device's `scratch`, looked up on the first call on
// the device (the current one); nullptr if the lookup fails.
void* device_scratch(int dev) {
  void* ptr = scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
    (void)hipGetLastError();
    return nullptr;
  }
  scratch_ptr[dev].store(ptr, std::memory_order_release);
  return ptr;
}

}  // namespace

extern "C" int qsdpa_forward_noalloc(const qsdpa_params* p, const void* q, const void* k, const void* v, void* o,
                                     void* stream) {
  const size_t need = qsdpa_workspace_bytes(p);
  if (need == 0) return qsdpa_validate_params(p);
  if (need > (size_t)QSDPA_SCRATCH_BYTES) return QSDPA_ERR_SCRATCH_TOO_SMALL;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return QSDPA_ERR_HIP;
  }
  void* ws = device_scratch(dev);
  if (!ws) return QSDPA_ERR_HIP;
  // every workspace byte the kernels read is written earlier in the same
  // call, so nothing needs clearing between calls
  return qsdpa::forward_impl(p, q, k, v, o, ws, (size_t)QSDPA_SCRATCH_BYTES, stream);
}
