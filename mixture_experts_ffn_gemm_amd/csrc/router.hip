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

constexpr int RL_JC = 64;  // router: j values per LDS chunk (two 32-blocks)

// Router logits for 4*RT tokens x 64 experts per workgroup (lane = expert, RT
// tokens per wavefront).  Each logit is one fp32 fused multiply-add chain over
// ascending j, from +0, then + bias (a separate fp32 add); the chain order is
// the contract that makes top-k ids reproducible bit for bit.  Per chunk of 64
// j the workgroup stages the transposed router slab (64 experts x 64 j) and the
// 4*RT token rows in LDS.  With one workgroup per CU the chunk loads are
// latency-bound, so they run PF chunks ahead through a ring of registers
// (the chunk loop is unrolled by PF so every ring slot is a fixed register).
// Zero padding past d leaves every chain unchanged (fma(0, 0, acc) = acc for
// acc != -0, and a chain from +0 never reaches -0).
//
// The workgroups of expert column 0 also run, on the staged x chunk, the
// per-32-block int8 quantiser (each 32-block is one half-wavefront) and the
// shared-expert gate dot product, so x is read from HBM once.
typedef float f4v __attribute__((ext_vector_type(4)));

template <int RT>
struct RouterChunk {
  f4v w[4];  // W rows jq = tid/64 + 4i of the chunk, expert = lane
  float x[RT];  // x[token tid/64 + 4r][chunk column lane]
};

struct RouterCtx {
  const f4v* wsrc;
  const float* xbase;
  int n, d, d4, d_pad, E64, t0, tid, lane, wave;
  bool quant;
  const float* shg;
  int8_t* xq;
  uint16_t* xs;
};

template <int RT>
__device__ __forceinline__ void router_fetch(RouterChunk<RT>& c, const RouterCtx& k, int ch) {
  const f4v z4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int jq = ch * (RL_JC / 4) + (k.tid >> 6) + 4 * i;
    c.w[i] = (jq < k.d4) ? k.wsrc[(size_t)jq * k.E64 + k.lane] : z4;
  }
  const int j = ch * RL_JC + k.lane;
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int t = min(k.t0 + (k.tid >> 6) + 4 * r, k.n - 1);
    c.x[r] = (j < k.d) ? k.xbase[(size_t)t * k.d + j] : 0.0f;
  }
}

// One chunk: stash the fetched slot into LDS buffer ch&1, refill the slot with
// chunk ch + PF, quantise (column-0 workgroups), run the fused chains.
template <int RT, int PF>
__device__ __forceinline__ void router_step(RouterChunk<RT>& slot, const RouterCtx& k, int ch, int nchunks,
                                            f4v (&wl)[2][RL_JC / 4][64], f4v (&xl)[2][4 * RT][RL_JC / 4],
                                            float (&acc)[RT], float (&gacc)[RT]) {
  constexpr int JQ = RL_JC / 4;
  const int buf = ch & 1;
#pragma unroll
  for (int i = 0; i < 4; ++i) wl[buf][(k.tid >> 6) + 4 * i][k.lane] = slot.w[i];
#pragma unroll
  for (int r = 0; r < RT; ++r)
    reinterpret_cast<float*>(&xl[buf][(k.tid >> 6) + 4 * r][0])[k.lane] = slot.x[r];
  lds_barrier();
  if (ch + PF < nchunks) router_fetch<RT>(slot, k, ch + PF);
  if (k.quant) {
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int tl = (k.tid >> 6) + 4 * r;
      const float val = reinterpret_cast<const float*>(&xl[buf][tl][0])[k.lane];
      const int j = ch * RL_JC + k.lane;
      int8_t q;
      uint16_t s16;
      quant_block32(val, q, s16);
      const int t = k.t0 + tl;
      if (t < k.n) {
        k.xq[(size_t)t * k.d_pad + j] = q;
        if ((k.lane & 31) == 0) k.xs[(size_t)t * (k.d_pad / QB) + (j >> 5)] = s16;
        if (k.shg && j < k.d) gacc[r] = __builtin_fmaf(val, k.shg[j], gacc[r]);
      }
    }
  }
  // LDS operands in batches of 4 f4v rows, then the fused chains
#pragma unroll
  for (int jb = 0; jb < JQ; jb += 4) {
    f4v wv[4], xv[RT][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) wv[q] = wl[buf][jb + q][k.lane];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int q = 0; q < 4; ++q) xv[r][q] = xl[buf][k.wave * RT + r][jb + q];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        acc[r] = __builtin_fmaf(xv[r][q].x, wv[q].x, acc[r]);
        acc[r] = __builtin_fmaf(xv[r][q].y, wv[q].y, acc[r]);
        acc[r] = __builtin_fmaf(xv[r][q].z, wv[q].z, acc[r]);
        acc[r] = __builtin_fmaf(xv[r][q].w, wv[q].w, acc[r]);
      }
  }
}

template <int RT>
__global__ __launch_bounds__(256, 1) void router_kernel(
    const float* __restrict__ x, int n, int d, int d_pad, const float* __restrict__ wt,
    const float* __restrict__ bias, int E, int E64, float* __restrict__ logits,
    const float* __restrict__ shg, float* __restrict__ gs, int8_t* __restrict__ xq,
    uint16_t* __restrict__ xs) {
  constexpr int TPW = 4 * RT;       // tokens per workgroup
  constexpr int JQ = RL_JC / 4;     // f4v rows per chunk
  constexpr int PF = 4;             // chunks in flight (one named register slot each)
  __shared__ f4v wl[2][JQ][64];
  __shared__ f4v xl[2][TPW][JQ];
  RouterCtx k;
  k.tid = threadIdx.x;
  k.lane = k.tid & 63;
  k.wave = __builtin_amdgcn_readfirstlane(k.tid >> 6);
  const int eg = blockIdx.y;
  k.quant = (eg == 0);
  k.t0 = blockIdx.x * TPW;
  k.n = n;
  k.d = d;
  k.d4 = d >> 2;
  k.d_pad = d_pad;
  k.E64 = E64;
  k.wsrc = reinterpret_cast<const f4v*>(wt) + eg * 64;
  k.xbase = x;
  k.shg = shg;
  k.xq = xq;
  k.xs = xs;
  const int e = eg * 64 + k.lane;

  float acc[RT], gacc[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    acc[r] = 0.0f;
    gacc[r] = 0.0f;
  }
  const int nchunks = (d + RL_JC - 1) / RL_JC;
  RouterChunk<RT> s0, s1, s2, s3;
  router_fetch<RT>(s0, k, 0);
  if (1 < nchunks) router_fetch<RT>(s1, k, 1);
  if (2 < nchunks) router_fetch<RT>(s2, k, 2);
  if (3 < nchunks) router_fetch<RT>(s3, k, 3);
  for (int ch0 = 0; ch0 < nchunks; ch0 += PF) {
    router_step<RT, PF>(s0, k, ch0, nchunks, wl, xl, acc, gacc);
    if (ch0 + 1 < nchunks) router_step<RT, PF>(s1, k, ch0 + 1, nchunks, wl, xl, acc, gacc);
    if (ch0 + 2 < nchunks) router_step<RT, PF>(s2, k, ch0 + 2, nchunks, wl, xl, acc, gacc);
    if (ch0 + 3 < nchunks) router_step<RT, PF>(s3, k, ch0 + 3, nchunks, wl, xl, acc, gacc);
  }
  if (e < E) {
    const float b = bias ? bias[e] : 0.0f;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int t = k.t0 + k.wave * RT + r;
      if (t < n) logits[(size_t)t * E + e] = bias ? acc[r] + b : acc[r];
    }
  }
  if (k.quant) {
    // zero blocks of the K padding not covered by the chunks
    const int jpad0 = nchunks * RL_JC;
    for (int v = k.tid; v < TPW * (d_pad - jpad0); v += 256) {
      const int tl = v / (d_pad - jpad0), j = jpad0 + v % (d_pad - jpad0);
      const int t = k.t0 + tl;
      if (t < n) {
        xq[(size_t)t * d_pad + j] = 0;
        if ((j & 31) == 0) xs[(size_t)t * (d_pad / QB) + (j >> 5)] = 0;
      }
    }
    if (shg) {
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        float a = gacc[r];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) a += __shfl_xor(a, off, 64);
        const int t = k.t0 + (k.tid >> 6) + 4 * r;
        if (k.lane == 0 && t < n) gs[t] = 1.0f / (1.0f + expf(-a));
      }
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
// wave-wide best-of-the-rest, softmax over all E, optional renormalisation;
// then wavefront 0 ranks the tile's (token, slot) pairs per expert in
// (token, slot) order and the tile's histogram is written for the bucketing
// kernel.
__global__ __launch_bounds__(256) void route_kernel(
    const float* __restrict__ logits, int n, int E, int k, int norm, int32_t* __restrict__ ids,
    float* __restrict__ wout, int32_t* __restrict__ rank, int32_t* __restrict__ hist) {
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

hipError_t launch_router(const float* x, int n, int d, int d_pad, const float* wt, const float* bias,
                         int E, int E64, float* logits, const float* sh_gate_vec, float* gs,
                         int8_t* xq, uint16_t* xs, hipStream_t s) {
  const int eg = E64 / 64;
  // tokens per wavefront: as many as keep >= 1024 wavefronts in flight
  int rt = 4;
  while (rt > 1 && (long)((n + rt - 1) / rt) * eg < 1024) rt >>= 1;
  dim3 grid((unsigned)((n + 4 * rt - 1) / (4 * rt)), (unsigned)eg);
  switch (rt) {
    case 4:
      router_kernel<4><<<grid, 256, 0, s>>>(x, n, d, d_pad, wt, bias, E, E64, logits, sh_gate_vec, gs, xq, xs);
      break;
    case 2:
      router_kernel<2><<<grid, 256, 0, s>>>(x, n, d, d_pad, wt, bias, E, E64, logits, sh_gate_vec, gs, xq, xs);
      break;
    default:
      router_kernel<1><<<grid, 256, 0, s>>>(x, n, d, d_pad, wt, bias, E, E64, logits, sh_gate_vec, gs, xq, xs);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_route(const float* logits, int n, int E, int k, int norm, int32_t* ids, float* w,
                        int32_t* rank, int32_t* hist, hipStream_t s) {
  const int tiles = (n + ROUTE_TILE - 1) / ROUTE_TILE;
  route_kernel<<<tiles, 256, 0, s>>>(logits, n, E, k, norm, ids, w, rank, hist);
  return hipGetLastError();
}

hipError_t launch_quantize(const float* v, int64_t n_values, int8_t* q, uint16_t* scales,
                           hipStream_t s) {
  const int64_t blocks = (n_values + 255) / 256;
  quantize_kernel<<<(unsigned)blocks, 256, 0, s>>>(v, n_values, q, scales);
  return hipGetLastError();
}

}  // namespace moe
