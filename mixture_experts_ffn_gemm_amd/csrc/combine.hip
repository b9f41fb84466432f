// combine.hip -- the ordered weighted combine and the layer-stack helper.
//
// SharpInference #129 "Scope": one launch over N x embDim that, for each token
// row, sums the na unweighted down-partials in top-k slot order (k = 0..na-1)
// with their per-(token, slot) weights, then adds the shared-expert row.  The
// per-token accumulation order is load-bearing, so every output element is one
// fp32 fused multiply-add chain in exactly that order.  The kernel is a pure
// stream (HBM-bound): each thread owns 4 consecutive columns of one token.
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
  float4 p[MAX_TOPK];
#pragma unroll
  for (int s = 0; s < MAX_TOPK; ++s)
    if (s < k) p[s] = pr[(size_t)s * d4];
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

// h += y (when y != NULL), then xn = h / sqrt(mean(h^2) + eps); one workgroup per row.
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

}  // namespace

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
  residual_rmsnorm_kernel<<<n, 256, 0, s>>>(h, y, xn, d, eps);
  return hipGetLastError();
}

}  // namespace moe
