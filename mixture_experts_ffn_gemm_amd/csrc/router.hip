// router.hip -- router logits, top-k / softmax / shared gate, per-32 int8
// activation quantiser and the per-tile expert histograms.
//
// SharpInference #388 "Remaining levers" 1 moves the router matvec
// norm[N x embDim] x routerW[numExperts x embDim] + softmax + top-k + shexp-gate
// onto the GPU; #408 "Hypothesis" lever 3 folds it into the GPU path for decode.
#include <hip/hip_fp16.h>

#include "device_util.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int RL_JC = 32;  // router: j values per LDS chunk (8 float4 rows)

// Logits for RT tokens per wavefront x 64 experts per workgroup column; lane =
// expert.  Each logit is one fp32 fused multiply-add chain over ascending j,
// from +0, then + bias (a separate fp32 add).  The chain order is the contract
// that makes top-k ids reproducible bit for bit.  The 64 x 32 slab of the
// transposed router matrix is staged in LDS once per workgroup and read by its
// four wavefronts; x comes in through wave-uniform (scalar) loads.
template <int RT>
__global__ __launch_bounds__(256) void router_logits_kernel(
    const float* __restrict__ x, int n, int d, const float* __restrict__ wt,
    const float* __restrict__ bias, int E, int E64, float* __restrict__ logits) {
  __shared__ float4 wl[2][RL_JC / 4][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int eg = blockIdx.y;
  const int t0 = blockIdx.x * 4 * RT + wave * RT;
  const int e = eg * 64 + lane;
  const float4* wsrc = reinterpret_cast<const float4*>(wt) + eg * 64;
  const float4* xr[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int t = min(t0 + r, n - 1);
    xr[r] = reinterpret_cast<const float4*>(x + (size_t)t * d);
  }
  float acc[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) acc[r] = 0.0f;

  const int nchunks = d / RL_JC;
  // cooperative load: 512 float4 per chunk, 2 per thread
  const int i0 = threadIdx.x, i1 = threadIdx.x + 256;
  float4 p0 = wsrc[(size_t)(i0 >> 6) * E64 + (i0 & 63)];
  float4 p1 = wsrc[(size_t)(i1 >> 6) * E64 + (i1 & 63)];
  wl[0][i0 >> 6][i0 & 63] = p0;
  wl[0][i1 >> 6][i1 & 63] = p1;
  __syncthreads();
  for (int ch = 0; ch < nchunks; ++ch) {
    const int buf = ch & 1;
    const bool more = ch + 1 < nchunks;
    if (more) {
      const size_t jq = (size_t)(ch + 1) * (RL_JC / 4);
      p0 = wsrc[(jq + (i0 >> 6)) * E64 + (i0 & 63)];
      p1 = wsrc[(jq + (i1 >> 6)) * E64 + (i1 & 63)];
    }
#pragma unroll
    for (int jl = 0; jl < RL_JC / 4; ++jl) {
      const float4 wv = wl[buf][jl][lane];
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        const float4 xv = xr[r][ch * (RL_JC / 4) + jl];
        acc[r] = __builtin_fmaf(xv.x, wv.x, acc[r]);
        acc[r] = __builtin_fmaf(xv.y, wv.y, acc[r]);
        acc[r] = __builtin_fmaf(xv.z, wv.z, acc[r]);
        acc[r] = __builtin_fmaf(xv.w, wv.w, acc[r]);
      }
    }
    if (more) {
      wl[buf ^ 1][i0 >> 6][i0 & 63] = p0;
      wl[buf ^ 1][i1 >> 6][i1 & 63] = p1;
    }
    __syncthreads();
  }
  if (e < E) {
    const float b = bias ? bias[e] : 0.0f;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int t = t0 + r;
      if (t < n) logits[(size_t)t * E + e] = bias ? acc[r] + b : acc[r];
    }
  }
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// a outranks b: higher logit, then lower id; id INT_MAX marks "no candidate".
__device__ inline bool outranks(float av, int ai, float bv, int bi) {
  if (ai == 0x7fffffff) return false;
  if (bi == 0x7fffffff) return true;
  return av > bv || (av == bv && ai < bi);
}

// One workgroup per 16 tokens, one wavefront per 4 of them: top-k by repeated
// wave-wide best-of-the-rest, softmax over all E, optional renormalisation,
// shared gate, int8 quantisation of x; then wavefront 0 ranks the tile's
// (token, slot) pairs per expert in (token, slot) order and the tile's
// histogram is written for the bucketing kernel.
__global__ __launch_bounds__(256) void route_kernel(
    const float* __restrict__ logits, const float* __restrict__ x, int n, int d, int d_pad, int E,
    int k, int norm, const float* __restrict__ shg, int32_t* __restrict__ ids,
    float* __restrict__ wout, float* __restrict__ gs, int32_t* __restrict__ rank,
    int8_t* __restrict__ xq, uint16_t* __restrict__ xs, int32_t* __restrict__ hist) {
  __shared__ int s_ids[ROUTE_TILE * MAX_TOPK];
  __shared__ int s_cnt[MAX_EXPERTS];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t0 = blockIdx.x * ROUTE_TILE;
  for (int e = threadIdx.x; e < E; e += 256) s_cnt[e] = 0;

  for (int i = 0; i < ROUTE_TILE / 4; ++i) {
    const int tl = wave * (ROUTE_TILE / 4) + i;
    const int t = t0 + tl;
    if (t >= n) break;
    float v[MAX_EXPERTS / 64];
    bool live[MAX_EXPERTS / 64];
#pragma unroll
    for (int c = 0; c < MAX_EXPERTS / 64; ++c) {
      const int e = lane + 64 * c;
      live[c] = e < E;
      v[c] = live[c] ? logits[(size_t)t * E + e] : 0.0f;
    }
    float m = 0.0f, myv = 0.0f;
    int myid = -1;
    for (int s = 0; s < k; ++s) {
      float bv = 0.0f;
      int bi = 0x7fffffff;
#pragma unroll
      for (int c = 0; c < MAX_EXPERTS / 64; ++c)
        if (live[c] && outranks(v[c], lane + 64 * c, bv, bi)) {
          bv = v[c];
          bi = lane + 64 * c;
        }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(bv, off, 64);
        const int oi = __shfl_xor(bi, off, 64);
        if (outranks(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
        }
      }
      if (s == 0) m = bv;
      if (lane == s) {
        myid = bi;
        myv = bv;
      }
#pragma unroll
      for (int c = 0; c < MAX_EXPERTS / 64; ++c)
        if (lane + 64 * c == bi) live[c] = false;
    }
    float part = 0.0f;
#pragma unroll
    for (int c = 0; c < MAX_EXPERTS / 64; ++c)
      if (lane + 64 * c < E) part += expf(v[c] - m);
    const float den = wave_sum(part);
    float p = (lane < k) ? expf(myv - m) / den : 0.0f;
    if (norm) {
      const float sum = wave_sum(p);
      p = p / sum;
    }
    if (lane < k) {
      ids[(size_t)t * k + lane] = myid;
      wout[(size_t)t * k + lane] = p;
      s_ids[tl * MAX_TOPK + lane] = myid;
    }
    const float* xt = x + (size_t)t * d;
    if (shg) {
      float a = 0.0f;
      for (int j = lane; j < d; j += 64) a = __builtin_fmaf(xt[j], shg[j], a);
      a = wave_sum(a);
      if (lane == 0) gs[t] = 1.0f / (1.0f + expf(-a));
    }
    for (int b2 = 0; b2 < d_pad / 64; ++b2) {
      const int j = b2 * 64 + lane;
      const float val = (j < d) ? xt[j] : 0.0f;
      int8_t q;
      uint16_t s16;
      quant_block32(val, q, s16);
      xq[(size_t)t * d_pad + j] = q;
      if ((lane & 31) == 0) xs[(size_t)t * (d_pad / QB) + 2 * b2 + (lane >> 5)] = s16;
    }
  }
  __syncthreads();
  if (wave == 0) {
    const int nt = min(ROUTE_TILE, n - t0);
    const int np = nt * k;
    for (int base = 0; base < np; base += 64) {
      const int q = base + lane;
      const bool valid = q < np;
      const int e = valid ? s_ids[(q / k) * MAX_TOPK + q % k] : -1;
      int r = 0;
      bool last = true;
      for (int i2 = 0; i2 < 64; ++i2) {
        const int ei = __builtin_amdgcn_readlane(e, i2);
        if (ei == e) {
          if (i2 < lane) ++r;
          if (i2 > lane) last = false;
        }
      }
      const int cbase = valid ? s_cnt[e] : 0;
      if (valid) rank[(size_t)(t0 + q / k) * k + q % k] = cbase + r;
      if (valid && last) s_cnt[e] = cbase + r + 1;
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) hist[(size_t)blockIdx.x * E + e] = s_cnt[e];
}

__global__ __launch_bounds__(256) void quantize_kernel(const float* __restrict__ v, int64_t n_values,
                                                       int8_t* __restrict__ q,
                                                       uint16_t* __restrict__ scales) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool valid = i < n_values;  // n_values % 32 == 0: a block is all valid or all not
  const float val = valid ? v[i] : 0.0f;
  int8_t qq;
  uint16_t s16;
  quant_block32(val, qq, s16);
  if (valid) {
    q[i] = qq;
    if ((threadIdx.x & 31) == 0) scales[i / QB] = s16;
  }
}

}  // namespace

hipError_t launch_router_logits(const float* x, int n, int d, const float* wt, const float* bias,
                                int E, int E64, float* logits, hipStream_t s) {
  const int eg = E64 / 64;
  // tokens per wavefront: as many as keep >= 1024 wavefronts in flight
  int rt = 4;
  while (rt > 1 && (long)((n + rt - 1) / rt) * eg < 1024) rt >>= 1;
  dim3 grid((unsigned)((n + 4 * rt - 1) / (4 * rt)), (unsigned)eg);
  switch (rt) {
    case 4: router_logits_kernel<4><<<grid, 256, 0, s>>>(x, n, d, wt, bias, E, E64, logits); break;
    case 2: router_logits_kernel<2><<<grid, 256, 0, s>>>(x, n, d, wt, bias, E, E64, logits); break;
    default: router_logits_kernel<1><<<grid, 256, 0, s>>>(x, n, d, wt, bias, E, E64, logits); break;
  }
  return hipGetLastError();
}

hipError_t launch_route(const float* logits, const float* x, int n, int d, int d_pad, int E, int k,
                        int norm, const float* sh_gate_vec, int32_t* ids, float* w, float* gs,
                        int32_t* rank, int8_t* xq, uint16_t* xs, int32_t* hist, hipStream_t s) {
  const int tiles = (n + ROUTE_TILE - 1) / ROUTE_TILE;
  route_kernel<<<tiles, 256, 0, s>>>(logits, x, n, d, d_pad, E, k, norm, sh_gate_vec, ids, w, gs,
                                     rank, xq, xs, hist);
  return hipGetLastError();
}

hipError_t launch_quantize(const float* v, int64_t n_values, int8_t* q, uint16_t* scales,
                           hipStream_t s) {
  const int64_t blocks = (n_values + 255) / 256;
  quantize_kernel<<<(unsigned)blocks, 256, 0, s>>>(v, n_values, q, scales);
  return hipGetLastError();
}

}  // namespace moe
