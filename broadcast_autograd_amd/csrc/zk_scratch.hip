// zk_scratch.hip -- the library-owned device scratch array behind
// zk_binary_bwd_noalloc: the workspace for callers that cannot allocate.
//
// `scratch` is a file-scope device array, so every GPU the library runs on
// holds its own copy of it until the process ends.  In host code the name
// `scratch` is only a host-side stand-in, never a device address: the
// device address of each GPU's copy comes from hipGetSymbolAddress, called
// once per device with that device current, and only that address is handed
// to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "zk.h"
#include "zk_kernels.h"

namespace zk {

static __device__ __align__(256) unsigned char scratch[ZK_SCRATCH_BYTES];

namespace {
constexpr int kMaxScratchDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void *ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_slots[kMaxScratchDevices];
}  // namespace

// The device address of the current device's scratch array (looked up on the
// device's first use, then cached).  hipErrorInvalidDevice past the table.
hipError_t scratch_on_current_device(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  ScratchSlot &s = g_slots[dev];
  std::call_once(s.once, [&s] {
    void *p = nullptr;
    s.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    s.ptr = s.err == hipSuccess ? p : nullptr;
  });
  if (s.err != hipSuccess) return s.err;
  *ptr = s.ptr;
  return hipSuccess;
}

}  // namespace zk
