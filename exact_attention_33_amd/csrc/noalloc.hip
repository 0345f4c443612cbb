// fa_fwd_noalloc: the forward of fa_fwd for callers that cannot allocate
// device memory.  The workspace fa_fwd takes from its caller (the split-KV
// path's partial results) comes instead from a static device array held by
// the library, one per GPU.  The contract is in include/fa_mi355x.h.
#include <mutex>

#include "fa_internal.h"

namespace {

constexpr size_t kScratchBytes = FA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte blocks");

// The library's scratch.  In host code this name is a host-side stand-in,
// not a device address: only the pointer resolved below reaches a kernel.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 256;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device, once resolved

// The device address of `scratch` on the current device, resolved on the
// first call with that device current and kept for later calls.
hipError_t scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" fa_status fa_fwd_noalloc(const void* q, const void* k, const void* v,
                                    const int32_t* kv_len, void* o, float* lse, fa_shape s,
                                    fa_dtype dtype, float scale, int causal, void* stream) {
  // The size check is host arithmetic only: a shape the scratch cannot hold
  // is turned away before any device call.
  const size_t need = fa_fwd_workspace_bytes(s, dtype, causal, nullptr);
  if (need > kScratchBytes)
    return fa::report_error(FA_ERR_WORKSPACE,
                            "fa_fwd_noalloc: this shape needs %zu bytes of scratch; the library's "
                            "static scratch holds %zu (use fa_fwd with a workspace)",
                            need, kScratchBytes);
  void* ws = nullptr;
  const hipError_t err = scratch_on_current_device(&ws);
  if (err != hipSuccess)
    return fa::report_error(FA_ERR_HIP, "fa_fwd_noalloc: cannot resolve the static scratch: %s",
                            hipGetErrorString(err));
  return fa_fwd(q, k, v, kv_len, o, lse, s, dtype, scale, causal, ws, kScratchBytes, stream);
}
