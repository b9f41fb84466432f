// noalloc.hip -- moe_ffn_prefill_static: the prefill entry point for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// The call is moe_ffn_prefill with the workspace taken from `scratch`, a
// file-scope device array of MOE_FFN_STATIC_SCRATCH_BYTES that the code
// object carries: every GPU the library runs on holds its own copy until the
// process ends.  In host code the array's name is only a host-side stand-in,
// so its device address is looked up once per device (hipGetSymbolAddress,
// with that device current) and only that address is ever handed to kernels.
//
// No part of the workspace has to start at zero (every stage writes what it
// reads), so nothing is cleared between calls.  All calls on one GPU share
// that GPU's array: calls that overlap in time on one GPU (two streams, two
// threads) race on it and must be serialised by the caller.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[MOE_FFN_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of each device's copy

// This device's copy of scratch, looked up on the first call on the device.
int scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_FFN_HIP_ERROR;
  if (dev < 0 || dev >= kMaxDevices) return MOE_FFN_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return MOE_FFN_HIP_ERROR;
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_FFN_OK;
}

}  // namespace

extern "C" int moe_ffn_prefill_static(const moe_ffn_weights* w, const float* x, int32_t n_tokens,
                                      float* out, const moe_ffn_routing* routing, hipStream_t stream) {
  if (!w || n_tokens < 0) return MOE_FFN_INVALID_ARG;
  size_t need = 0;
  const int rc = moe_ffn_workspace_size(w, n_tokens, &need);
  if (rc != MOE_FFN_OK) return rc;
  if (need > (size_t)MOE_FFN_STATIC_SCRATCH_BYTES) return MOE_FFN_SCRATCH_TOO_SMALL;
  void* ws = nullptr;
  const int src = scratch_for_current_device(&ws);
  if (src != MOE_FFN_OK) return src;
  return moe_ffn_prefill(w, x, n_tokens, out, ws, (size_t)MOE_FFN_STATIC_SCRATCH_BYTES, routing, stream);
}
