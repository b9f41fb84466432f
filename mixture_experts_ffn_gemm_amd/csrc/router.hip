// router.hip -- router logits, top-k / softmax, the per-tile expert
// histograms, and the per-32 int8 activation quantiser (with the shared gate),
// which runs after the bucketing and scatters each token's codes to its
// expert slots.
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
typedef float f4v __attribute__((ext_vector_type(4)));

template <int RT>
struct RouterChunk {
  f4v w[4];  // W rows jq = tid/64 + 4i of the chunk, expert = lane
  float x[RT];  // x[token tid/64 + 4r][chunk column lane]
};

struct RouterCtx {
  const f4v* wsrc;
  const float* xbase;
  int n, d, d4, E64, t0, tid, lane, wave;
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
// chunk ch + PF, run the fused chains.
template <int RT, int PF>
__device__ __forceinline__ void router_step(RouterChunk<RT>& slot, const RouterCtx& k, int ch, int nchunks,
                                            f4v (&wl)[2][RL_JC / 4][64], f4v (&xl)[2][4 * RT][RL_JC / 4],
                                            float (&acc)[RT]) {
  constexpr int JQ = RL_JC / 4;
  const int buf = ch & 1;
#pragma unroll
  for (int i = 0; i < 4; ++i) wl[buf][(k.tid >> 6) + 4 * i][k.lane] = slot.w[i];
#pragma unroll
  for (int r = 0; r < RT; ++r)
    reinterpret_cast<float*>(&xl[buf][(k.tid >> 6) + 4 * r][0])[k.lane] = slot.x[r];
  lds_barrier();
  if (ch + PF < nchunks) router_fetch<RT>(slot, k, ch + PF);
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
    const float* __restrict__ x, int n, int d, const float* __restrict__ wt,
    const float* __restrict__ bias, int E, int E64, float* __restrict__ logits) {
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
  k.t0 = blockIdx.x * TPW;
  k.n = n;
  k.d = d;
  k.d4 = d >> 2;
  k.E64 = E64;
  k.wsrc = reinterpret_cast<const f4v*>(wt) + eg * 64;
  k.xbase = x;
  const int e = eg * 64 + k.lane;

  float acc[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) acc[r] = 0.0f;
  const int nchunks = (d + RL_JC - 1) / RL_JC;
  RouterChunk<RT> s0, s1, s2, s3;
  router_fetch<RT>(s0, k, 0);
  if (1 < nchunks) router_fetch<RT>(s1, k, 1);
  if (2 < nchunks) router_fetch<RT>(s2, k, 2);
  if (3 < nchunks) router_fetch<RT>(s3, k, 3);
  for (int ch0 = 0; ch0 < nchunks; ch0 += PF) {
    router_step<RT, PF>(s0, k, ch0, nchunks, wl, xl, acc);
    if (ch0 + 1 < nchunks) router_step<RT, PF>(s1, k, ch0 + 1, nchunks, wl, xl, acc);
    if (ch0 + 2 < nchunks) router_step<RT, PF>(s2, k, ch0 + 2, nchunks, wl, xl, acc);
    if (ch0 + 3 < nchunks) router_step<RT, PF>(s3, k, ch0 + 3, nchunks, wl, xl, acc);
  }
  if (e < E) {
    const float b = bias ? bias[e] : 0.0f;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int t = k.t0 + k.wave * RT + r;
      if (t < n) logits[(size_t)t * E + e] = bias ? acc[r] + b : acc[r];
    }
  }
}

// Activation quantiser and scatter, after the bucketing: one wavefront per
// token row.  Lane pairs quantise 32-blocks (each lane 16 values), and each
// block's codes and scale are written once per expert slot of the token,
// straight into the GEMM operand layout at the slot's padded row
// (t32 = row / 32, r = row % 32): one 4 KiB slab per (t32, k-step) holding
// [32 rows][128 B], piece p (16 codes: block p/2 of the k-step, half p%2)
// of row r at 16 * (p ^ (r % 8)), and the scales at [t32][k-step][r][block].
// The 8 lanes of one k-step therefore write one whole 128-byte line per slot.
// The K-padding blocks past d get zero codes and scales.  With a shared
// expert the wavefront also computes the gate sigmoid(x . g) (a fixed-order
// reduction).  Optionally the token-major codes and scales are written out.
__global__ __launch_bounds__(256) void quantize_scatter_kernel(
    const float* __restrict__ x, int n, int d, int d_pad, const int32_t* __restrict__ pos, int kk,
    int pad_rows, int8_t* __restrict__ gq, uint16_t* __restrict__ gqs,
    const float* __restrict__ shg, float* __restrict__ gs, int8_t* __restrict__ xq_out,
    uint16_t* __restrict__ xs_out) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= n) return;
  const float* xr = x + (size_t)t * d;
  const int KS = d_pad / (QB * KSTEP);
  int prow[MAX_TOPK + 1];
#pragma unroll
  for (int s = 0; s < MAX_TOPK + 1; ++s) {
    const int v = s < kk ? pos[(size_t)t * kk + s] : -1;
    prow[s] = (v >= 0 && v < pad_rows) ? v : -1;
  }
  float gacc = 0.0f;
  for (int j0 = 0; j0 < KS; j0 += 8) {
    const int j = j0 + (lane >> 3), p = lane & 7;  // k-step, piece
    const int kb = KSTEP * j + (p >> 1), half = p & 1;
    const int c0 = kb * QB + half * 16;  // first column of the piece
    float v[16];
    if (c0 < d) {  // d % 32 == 0: a piece is all valid or all padding
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 q = *reinterpret_cast<const float4*>(xr + c0 + 4 * i);
        v[4 * i] = q.x;
        v[4 * i + 1] = q.y;
        v[4 * i + 2] = q.z;
        v[4 * i + 3] = q.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = 0.0f;
    }
    uint32_t pk[4];
    uint16_t s16;
    quant_half_block16(v, pk, s16);  // lanes 2i, 2i+1 share a block; all take part
    if (j < KS) {
      const uint4 codes = make_uint4(pk[0], pk[1], pk[2], pk[3]);
#pragma unroll
      for (int s = 0; s < MAX_TOPK + 1; ++s) {
        const int row = prow[s];
        if (s < kk && row >= 0) {
          const int t32 = row >> 5, r = row & 31;
          const size_t slab = (size_t)t32 * KS + j;
          *reinterpret_cast<uint4*>(gq + (slab * 32 + r) * 128 + ((p ^ (r & 7)) << 4)) = codes;
          if (half == 0) gqs[(slab * 32 + r) * KSTEP + (p >> 1)] = s16;
        }
      }
      if (xq_out && c0 < d) *reinterpret_cast<uint4*>(xq_out + (size_t)t * d + c0) = codes;
      if (xs_out && half == 0 && c0 < d) xs_out[(size_t)t * (d / QB) + kb] = s16;
    }
    if (shg && c0 < d) {
#pragma unroll
      for (int i = 0; i < 16; ++i) gacc = __builtin_fmaf(v[i], shg[c0 + i], gacc);
    }
  }
  if (shg) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) gacc += __shfl_xor(gacc, off, 64);
    if (lane == 0) gs[t] = 1.0f / (1.0f + expf(-gacc));
  }
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// One workgroup per 16 tokens.  The tile's logits are staged in LDS; each
// (token, expert) finds its rank among the token's experts -- the number of
// experts with a larger logit, or an equal logit and a lower id -- and the
// experts of rank < k take slot = rank.  This is the top-k of the contract
// (logit descending, id ascending) computed without any serial reduction.
// Then softmax over all E, optional renormalisation, and the per-expert rank
// of each (token, slot) pair among the tile's pairs in (token, slot) order,
// with the tile's histogram, for the bucketing kernel.
__global__ __launch_bounds__(256) void route_kernel(
    const float* __restrict__ logits, int n, int E, int k, int norm, int32_t* __restrict__ ids,
    float* __restrict__ wout, int32_t* __restrict__ rank, int32_t* __restrict__ hist) {
  __shared__ __attribute__((aligned(16))) float s_l[ROUTE_TILE][MAX_EXPERTS + 4];
  __shared__ __attribute__((aligned(16))) int s_ids[ROUTE_TILE * MAX_TOPK];
  __shared__ float s_val[ROUTE_TILE][MAX_TOPK];
  __shared__ int s_cnt[MAX_EXPERTS];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * ROUTE_TILE;
  const int nt = min(ROUTE_TILE, n - t0);
  for (int i = tid; i < ROUTE_TILE * E; i += 256) {
    const int tl = i / E, e = i - tl * E;
    s_l[tl][e] = (tl < nt) ? logits[(size_t)(t0 + tl) * E + e] : 0.0f;
  }
  if (E & 3)  // pad each row to a multiple of 4 with -inf
    for (int i = tid; i < ROUTE_TILE * 4; i += 256) {
      const int tl = i >> 2, e = E + (i & 3);
      if (e < ((E + 3) & ~3)) s_l[tl][e] = -__builtin_huge_valf();
    }
  for (int e = tid; e < E; e += 256) s_cnt[e] = 0;
  __syncthreads();

  // ranks: thread (token tl = tid/16, expert group g = tid%16) owns experts g + 16c
  const int tl = tid >> 4, g = tid & 15;
  const int E4 = (E + 3) & ~3;  // logits row padded to 4 with -inf (never outranks)
  for (int e = g; e < E; e += 16) {
    const float le = s_l[tl][e];
    int r = 0;
#pragma unroll 4
    for (int e2 = 0; e2 < E4; e2 += 4) {
      const float4 l4 = *reinterpret_cast<const float4*>(&s_l[tl][e2]);
      r += (l4.x > le || (l4.x == le && e2 + 0 < e)) ? 1 : 0;
      r += (l4.y > le || (l4.y == le && e2 + 1 < e)) ? 1 : 0;
      r += (l4.z > le || (l4.z == le && e2 + 2 < e)) ? 1 : 0;
      r += (l4.w > le || (l4.w == le && e2 + 3 < e)) ? 1 : 0;
    }
    if (r < k) {
      s_ids[tl * MAX_TOPK + r] = e;
      s_val[tl][r] = le;
    }
  }
  __syncthreads();

  // softmax over all E (the 16 threads of a token share the sum), weights of the k slots
  const float m = s_val[tl][0];
  float part = 0.0f;
  for (int e = g; e < E; e += 16) part += expf(s_l[tl][e] - m);
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) part += __shfl_xor(part, off, 16);
  float p = (g < k) ? expf(s_val[tl][min(g, k - 1)] - m) / part : 0.0f;
  if (norm) {
    float sum = p;
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 16);
    p = p / sum;
  }
  if (tl < nt && g < k) {
    ids[(size_t)(t0 + tl) * k + g] = s_ids[tl * MAX_TOPK + g];
    wout[(size_t)(t0 + tl) * k + g] = p;
  }

  // rank of pair q = (token, slot) among the tile's earlier pairs of the same expert
  const int np = nt * k;
  if (tid < np) {
    const int q = tid;
    const int e = s_ids[(q / k) * MAX_TOPK + q % k];
    int r = 0;
    bool last = true;
    // pairs of earlier tokens (all their k slots), then this token's earlier slots
    for (int t2 = 0; t2 < nt; ++t2) {
      const int4* row = reinterpret_cast<const int4*>(&s_ids[t2 * MAX_TOPK]);
#pragma unroll
      for (int c4 = 0; c4 < MAX_TOPK / 4; ++c4) {
        if (4 * c4 >= k) break;
        const int4 v = row[c4];
        const int ev[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int s2 = 4 * c4 + u;
          if (s2 < k && ev[u] == e) {
            const int q2 = t2 * k + s2;
            r += (q2 < q) ? 1 : 0;
            if (q2 > q) last = false;
          }
        }
      }
    }
    rank[(size_t)(t0 + q / k) * k + q % k] = r;
    if (last) s_cnt[e] = r + 1;
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) hist[(size_t)blockIdx.x * E + e] = s_cnt[e];
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

hipError_t launch_router(const float* x, int n, int d, const float* wt, const float* bias, int E,
                         int E64, float* logits, hipStream_t s) {
  const int eg = E64 / 64;
  // tokens per wavefront: as many as keep >= 1024 wavefronts in flight
  int rt = 4;
  while (rt > 1 && (long)((n + rt - 1) / rt) * eg < 1024) rt >>= 1;
  dim3 grid((unsigned)((n + 4 * rt - 1) / (4 * rt)), (unsigned)eg);
  switch (rt) {
    case 4: router_kernel<4><<<grid, 256, 0, s>>>(x, n, d, wt, bias, E, E64, logits); break;
    case 2: router_kernel<2><<<grid, 256, 0, s>>>(x, n, d, wt, bias, E, E64, logits); break;
    default: router_kernel<1><<<grid, 256, 0, s>>>(x, n, d, wt, bias, E, E64, logits); break;
  }
  return hipGetLastError();
}

hipError_t launch_quantize_scatter(const float* x, int n, int d, int d_pad, const int32_t* pos,
                                  int kk, int pad_rows, int8_t* gq, uint16_t* gqs,
                                  const float* sh_gate_vec, float* gs, int8_t* xq_out,
                                  uint16_t* xs_out, hipStream_t s) {
  quantize_scatter_kernel<<<(n + 3) / 4, 256, 0, s>>>(x, n, d, d_pad, pos, kk, pad_rows, gq, gqs,
                                                      sh_gate_vec, gs, xq_out, xs_out);
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
