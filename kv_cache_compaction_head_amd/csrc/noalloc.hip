// kvc_compact without a caller workspace: the workspace is a file-scope
// device array of KVC_NOALLOC_SCRATCH_BYTES, so the call allocates nothing
// (for code under HIP graph capture, tight serving loops and other callers
// that cannot call hipMalloc).
//
// Each device the library runs on holds its own copy of the array until the
// process ends.  Its device address is taken once per device, with that
// device current, by hipGetSymbolAddress; host code only ever passes that
// address on (the array's name in host code is a host-side stand-in, not a
// device address).  Every call on a device shares its array, so calls that
// overlap in time on one device race; the kernels clear what must start at
// zero (status words, team barrier words) on every call, as they do for a
// caller's workspace.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/kvc.h"

namespace {

static __device__ __align__(256) unsigned char scratch[KVC_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch`, per device
std::mutex g_scratch_mu;

// The current device's address of the array (looked up on its first use on
// that device), or null if HIP cannot provide it.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int kvc_compact_noalloc(const kvc_params_t* p, const void* Q_ref, const void* K,
                                   const void* V, void* out_K, float* out_bias, void* out_V,
                                   int32_t* out_idx, int32_t* out_status, hipStream_t stream) {
  const size_t need = kvc_workspace_bytes(p);
  if (need == 0) return KVC_EINVAL;
  if (need > KVC_NOALLOC_SCRATCH_BYTES) return KVC_EWORKSPACE;
  void* ws = scratch_ptr();
  if (!ws) return KVC_EHIP;
  return kvc_compact(p, Q_ref, K, V, out_K, out_bias, out_V, out_idx, out_status, ws,
                     KVC_NOALLOC_SCRATCH_BYTES, stream);
}
