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

// The same quantiser with each lane holding half a block (16 values; lanes
// 2i and 2i+1 hold block i): amax over the lane pair, then the codes of this
// lane's 16 values packed little-endian into 4 words.  Decisions identical to
// quant_block32.
__device__ inline void quant_half_block16(const float (&v)[16], uint32_t (&packed)[4],
                                          uint16_t& s16) {
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(v[i]));
  a = fmaxf(a, __shfl_xor(a, 1, 64));
  if (a == 0.0f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) packed[i] = 0u;
    s16 = 0;
    return;
  }
  const float dd = a / 127.0f;
  const float id = 127.0f / a;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t w = 0u;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      float r = rintf(v[4 * i + b] * id);
      r = fminf(fmaxf(r, -127.0f), 127.0f);
      w |= ((uint32_t)(int)r & 0xffu) << (8 * b);
    }
    packed[i] = w;
  }
  s16 = __half_as_ushort(__float2half_rn(dd));
}

// A 64-bit key per (logit, expert id) whose unsigned order is the top-k order
// (logit descending, then id ascending): the float's bits mapped to an
// unsigned order (-0 taken as +0, so that equal logits tie as in a float
// comparison) above the inverted id.  Every real key is > 0.
__device__ __forceinline__ unsigned long long topk_key(float l, int e) {
  const uint32_t b = l == 0.0f ? 0u : __float_as_uint(l);
  const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((unsigned long long)ord << 32) | (uint32_t)~(uint32_t)e;
}

// Wavefront maximum of an unsigned value: prefix maxima within each row of
// 16 lanes by DPP shifts, the row maxima carried into rows 1 and 3, then into
// rows 2 and 3 by DPP row broadcasts; lane 63 ends with the maximum, which is
// returned to every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true));  // row_shr:1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true));  // row_shr:2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true));  // row_shr:4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true));  // row_shr:8
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));  // row_bcast:15
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return __builtin_amdgcn_readlane(v, 63);
}

// Wavefront maximum of 64-bit keys whose values are distinct across lanes (or
// zero): the maximum of the high words, then of the low words among the lanes
// that hold that high word.
__device__ __forceinline__ unsigned long long wave_max_key(unsigned long long v) {
  const uint32_t mh = wave_max_u32((uint32_t)(v >> 32));
  const uint32_t ml = wave_max_u32((uint32_t)(v >> 32) == mh ? (uint32_t)v : 0u);
  return ((unsigned long long)mh << 32) | ml;
}

// Workgroup barrier that orders LDS accesses only: global loads still in flight
// (a register prefetch ring) are not drained, unlike __syncthreads().
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace moe
