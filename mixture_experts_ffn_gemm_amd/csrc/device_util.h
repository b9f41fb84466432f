// device_util.h -- small device helpers shared by the kernels of libmoe_ffn.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Per-32-block int8 quantiser over one half-wavefront (32 lanes = one block,
// each lane holds one value).  Every decision is fp32: amax, 127/amax, the
// product, round-half-even; the scale is binary16(amax/127); a zero block gives
// zero codes and a zero scale.  (SharpInference #408 "Hypothesis" lever 2:
// int8 block activations for the expert matvec.)
__device__ inline void quant_block32(float v, int8_t& q, uint16_t& s16) {
  float a = fabsf(v);
#pragma unroll
  for (int off = 16; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
  if (a == 0.0f) {
    q = 0;
    s16 = 0;
    return;
  }
  const float dd = a / 127.0f;
  const float id = 127.0f / a;
  float r = rintf(v * id);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  q = (int8_t)(int)r;
  s16 = __half_as_ushort(__float2half_rn(dd));
}


// Workgroup barrier that orders LDS accesses only: global loads still in flight
// (a register prefetch ring) are not drained, unlike __syncthreads().
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace moe
