// The forward for callers that cannot allocate device memory: the workspace of
// magi_attn_fwd (the K-hat / V^T tile images of the bf16 path, the partial
// results of split items and the per-item softmax flags) comes from a static
// device array instead of the caller.
//
// `scratch` holds kNoAllocScratchBytes on every GPU the library runs on, for
// the life of the process. In host code its name stands for a host-side
// shadow, not a device address, so the array's device address is taken once
// per device with hipGetSymbolAddress (that device current) and only that
// address is handed to the kernels. Calls on one GPU share its array: the
// forward overwrites every byte it later reads (images, partials and flags
// are written before they are read within a call), so nothing needs clearing
// between calls, but calls that overlap in time on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "kernels.hpp"
#include "magi_attn.h"

namespace {

constexpr size_t kNoAllocScratchBytes = size_t(MAGI_ATTN_NOALLOC_SCRATCH_BYTES);
static_assert(kNoAllocScratchBytes % 256 == 0, "scratch size");

__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};       // device address of `scratch` on each device, once known

// Device address of this device's scratch array (the device must be current).
hipError_t scratch_address(int dev, void** ptr) {
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

MAGI_API magi_status_t magi_attn_fwd_noalloc(const magi_attn_plan_t* plan, const void* q, const void* k,
                                             const void* v, const float* q_gain, const float* k_gain,
                                             float rms_eps, float scale, void* out, float* lse, void* stream) {
  size_t need = 0;
  magi_status_t s = magi_attn_workspace_size(plan, &need);
  if (s != MAGI_OK) return s;
  if (need > kNoAllocScratchBytes)
    return magi::set_last_error(MAGI_ERR_UNSUPPORTED,
                                "the plan's workspace (" + std::to_string(need) + " bytes) exceeds the static scratch "
                                "of magi_attn_fwd_noalloc (" + std::to_string(kNoAllocScratchBytes) +
                                " bytes): use magi_attn_fwd with a caller workspace");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return magi::set_last_error(MAGI_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return magi::set_last_error(MAGI_ERR_UNSUPPORTED, "device index out of range");
  void* ws = nullptr;
  e = scratch_address(dev, &ws);
  if (e != hipSuccess)
    return magi::set_last_error(MAGI_ERR_HIP, std::string("hipGetSymbolAddress of the scratch array: ") +
                                              hipGetErrorString(e));
  return magi_attn_fwd(plan, q, k, v, q_gain, k_gain, rms_eps, scale, out, lse, ws, kNoAllocScratchBytes, stream);
}

}  // extern "C"
