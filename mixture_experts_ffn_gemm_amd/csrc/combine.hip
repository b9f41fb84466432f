// combine.hip -- the ordered weighted combine and the layer-stack helper.
//
// SharpInference #129, "Scope": a single launch covers all N x d outputs.
// Output element (t, j) is an fp32 fused multiply-add chain that starts at +0,
// takes slot 0, 1, ..., k-1 of token t (weight times unweighted partial) and
// ends with the gated shared-expert row.  Results must not depend on how the
// work is split, so that chain order is fixed.  The kernel is a pure stream
// (HBM-bound): each thread owns 4 consecutive columns of one token.
#include "internal.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void combine_kernel(const float4* __restrict__ partial,
                                                     const float* __restrict__ w,
                                                     const float* __restrict__ gs, int n, int k,
                                                     int kk, int d4, float4* __restrict__ out) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long)n * d4) return;
  const int t = (int)(i / d4);
  const int j = (int)(i - (long)t * d4);
  const float4* pr = partial + (size_t)t * kk * d4 + j;
  // the partials are read once: non-temporal loads
  typedef float f4n __attribute__((ext_vector_type(4)));
  float4 p[MAX_TOPK];
#pragma unroll
  for (int s = 0; s < MAX_TOPK; ++s)
    if (s < k) {
      const f4n v = __builtin_nontemporal_load(reinterpret_cast<const f4n*>(pr + (size_t)s * d4));
      p[s] = make_float4(v.x, v.y, v.z, v.w);
    }
  float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
  for (int s = 0; s < MAX_TOPK; ++s)
    if (s < k) {
      const float ws = w[(size_t)t * k + s];
      o.x = __builtin_fmaf(ws, p[s].x, o.x);
      o.y = __builtin_fmaf(ws, p[s].y, o.y);
      o.z = __builtin_fmaf(ws, p[s].z, o.z);
      o.w = __builtin_fmaf(ws, p[s].w, o.w);
    }
  if (gs) {
    const float g = gs[t];
    const float4 q = pr[(size_t)k * d4];
    o.x = __builtin_fmaf(g, q.x, o.x);
    o.y = __builtin_fmaf(g, q.y, o.y);
    o.z = __builtin_fmaf(g, q.z, o.z);
    o.w = __builtin_fmaf(g, q.w, o.w);
  }
  out[i] = o;
}

// h += y (when y != NULL), then xn = h / sqrt(mean(h^2) + eps); one workgroup
// per row.  This form serves rows whose length is not a multiple of 4.
__global__ __launch_bounds__(256) void residual_rmsnorm_kernel(float* __restrict__ h,
                                                               const float* __restrict__ y,
                                                               float* __restrict__ xn, int d,
                                                               float eps) {
  __shared__ float s_part[4];
  const int t = blockIdx.x;
  float* hr = h + (size_t)t * d;
  const float* yr = y ? y + (size_t)t * d : nullptr;
  float ss = 0.0f;
  for (int j = threadIdx.x; j < d; j += 256) {
    float v = hr[j];
    if (yr) {
      v = v + yr[j];
      hr[j] = v;
    }
    ss = __builtin_fmaf(v, v, ss);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (s_part[0] + s_part[1]) + (s_part[2] + s_part[3]);
  const float r = 1.0f / sqrtf(tot / (float)d + eps);
  for (int j = threadIdx.x; j < d; j += 256) xn[(size_t)t * d + j] = hr[j] * r;
}

// The residual add and RMSNorm of one row of d = 4 * d4 values, h += y and
// xn = h / sqrt(mean(h^2) + eps), where y is
//   COMBINE: the ordered combine of the row's partials (per element the
//            chain of combine_kernel), never stored;
//   else:    the y row, or nothing when y == NULL.
// Thread i owns the 4-column chunks i, i + 256, ...; it accumulates the
// squares chunk by chunk (x, y, z, w), the wavefronts reduce by xor
// shuffles and the 4 wavefront sums meet in a fixed order.  The two forms
// therefore give h and xn bit for bit alike: the stack's fused layer equals
// the plain layer followed by the plain helper.  xn may be the layer's own
// input in the fused form (every read of it happened in earlier kernels).
// One workgroup per row; all loads of a chunk are issued before its math.
template <bool COMBINE>
__global__ __launch_bounds__(256) void residual_rmsnorm4_kernel(
    const float4* __restrict__ partial, const float* __restrict__ w, const float* __restrict__ gs,
    int k, int kk, const float4* __restrict__ y, int d4, float4* __restrict__ h,
    float4* __restrict__ xn, float eps) {
  __shared__ float s_part[4];
  const int t = blockIdx.x;
  float4* hr = h + (size_t)t * d4;
  const float4* pr = COMBINE ? partial + (size_t)t * kk * d4 : nullptr;
  const float4* yr = (!COMBINE && y) ? y + (size_t)t * d4 : nullptr;
  float ws[MAX_TOPK];
  float g = 0.0f;
  if constexpr (COMBINE) {
#pragma unroll
    for (int s = 0; s < MAX_TOPK; ++s) ws[s] = (s < k) ? w[(size_t)t * k + s] : 0.0f;
    if (gs) g = gs[t];
  }
  float ss = 0.0f;
#pragma unroll 2
  for (int c = threadIdx.x; c < d4; c += 256) {
    float4 v = hr[c];
    float4 o;
    bool add = true;
    if constexpr (COMBINE) {
      float4 p[MAX_TOPK + 1];
#pragma unroll
      for (int s = 0; s < MAX_TOPK; ++s)
        if (s < k) p[s] = pr[(size_t)s * d4 + c];
      if (gs) p[MAX_TOPK] = pr[(size_t)k * d4 + c];
      o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
      for (int s = 0; s < MAX_TOPK; ++s)
        if (s < k) {
          o.x = __builtin_fmaf(ws[s], p[s].x, o.x);
          o.y = __builtin_fmaf(ws[s], p[s].y, o.y);
          o.z = __builtin_fmaf(ws[s], p[s].z, o.z);
          o.w = __builtin_fmaf(ws[s], p[s].w, o.w);
        }
      if (gs) {
        o.x = __builtin_fmaf(g, p[MAX_TOPK].x, o.x);
        o.y = __builtin_fmaf(g, p[MAX_TOPK].y, o.y);
        o.z = __builtin_fmaf(g, p[MAX_TOPK].z, o.z);
        o.w = __builtin_fmaf(g, p[MAX_TOPK].w, o.w);
      }
    } else if (yr) {
      o = yr[c];
    } else {
      add = false;
    }
    if (add) {
      v.x = v.x + o.x;
      v.y = v.y + o.y;
      v.z = v.z + o.z;
      v.w = v.w + o.w;
      hr[c] = v;
    }
    ss = __builtin_fmaf(v.x, v.x, ss);
    ss = __builtin_fmaf(v.y, v.y, ss);
    ss = __builtin_fmaf(v.z, v.z, ss);
    ss = __builtin_fmaf(v.w, v.w, ss);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (s_part[0] + s_part[1]) + (s_part[2] + s_part[3]);
  const float r = 1.0f / sqrtf(tot / (float)(4 * d4) + eps);
  float4* xr = xn + (size_t)t * d4;
  for (int c = threadIdx.x; c < d4; c += 256) {
    const float4 v = hr[c];
    xr[c] = make_float4(v.x * r, v.y * r, v.z * r, v.w * r);
  }
}

}  // namespace

hipError_t launch_combine_residual_rmsnorm(const float* partial, const float* w, const float* gs, int n,
                                           int k, int kk, int d, float* h, float* xn, float eps,
                                           hipStream_t s) {
  // d % 32 == 0 for a layer
  residual_rmsnorm4_kernel<true><<<n, 256, 0, s>>>(reinterpret_cast<const float4*>(partial), w, gs, k, kk,
                                                   nullptr, d / 4, reinterpret_cast<float4*>(h),
                                                   reinterpret_cast<float4*>(xn), eps);
  return hipGetLastError();
}

hipError_t launch_combine(const float* partial, const float* w, const float* gs, int n, int k,
                          int kk, int d, float* out, hipStream_t s) {
  const int d4 = d / 4;
  const long total = (long)n * d4;
  combine_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(
      reinterpret_cast<const float4*>(partial), w, gs, n, k, kk, d4, reinterpret_cast<float4*>(out));
  return hipGetLastError();
}

hipError_t launch_residual_rmsnorm(float* h, const float* y, float* xn, int n, int d, float eps,
                                   hipStream_t s) {
  const bool v4 = d % 4 == 0 && !((uintptr_t)h & 15u) && !((uintptr_t)xn & 15u) && !((uintptr_t)y & 15u);
  if (v4)
    residual_rmsnorm4_kernel<false><<<n, 256, 0, s>>>(nullptr, nullptr, nullptr, 0, 0,
                                                      reinterpret_cast<const float4*>(y), d / 4,
                                                      reinterpret_cast<float4*>(h),
                                                      reinterpret_cast<float4*>(xn), eps);
  else
    residual_rmsnorm_kernel<<<n, 256, 0, s>>>(h, y, xn, d, eps);
  return hipGetLastError();
}

}  // namespace moe
