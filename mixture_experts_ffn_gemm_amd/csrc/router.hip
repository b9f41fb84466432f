// router.hip -- router logits, top-k / softmax, the per-tile expert
// histograms, the decode router, and the standalone per-32 int8 quantiser.
// (The prefill activation quantiser runs in the bucketing launch.)
//
// The routing step of the layer runs on the device for prefill
// (SharpInference #388, "Remaining levers" 1) and for decode (#408,
// "Hypothesis" lever 3): every token's logits against every expert row, the
// softmax, the top-k selection and the shared-expert gate.
#include <hip/hip_fp16.h>

#include "device_util.h"
#include "internal.h"

namespace moe {
namespace {

typedef float f4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int RJC = 64;          // router: j values per LDS chunk
constexpr int RJQ = RJC / 4;     // 4-j quads per chunk
// chunk buffers in the LDS ring: 6 (108 KiB, one workgroup per CU) when every
// workgroup of the launch fits on the chip at once, else 3 (54 KiB, two
// workgroups per CU, so a second round of workgroups never waits for a whole
// first round; the shallower ring costs the single-round case ~1.5 us)
constexpr int RNB_DEEP = 6;
constexpr int RNB_SHALLOW = 3;
constexpr int RDMA = 3;          // copies per wavefront per chunk
constexpr int RT = 1;            // tokens per wavefront
constexpr int RW = 8;            // wavefronts per workgroup
constexpr int R_WB = RJQ * 64 * 16;       // transposed router slab per chunk (16 KiB)
constexpr int R_XB = RW * RT * RJC * 4;   // the workgroup's token rows per chunk (2 KiB)
constexpr int R_BUF = R_WB + R_XB;
static_assert(RJQ == 2 * RW && RDMA == 3, "each wavefront copies two slab quads and its token row per chunk");

// global -> LDS copies: lane l writes LDS address m0 + size * l
__device__ __forceinline__ void rdma16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void rdma4(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void rwait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// 16 steps of one fp32 fused multiply-add chain: for i = 0..15,
//   acc0 = fma(xa[i], w[i], acc0),
// where xa[i] is lane i of this lane's 16-lane row of xa, broadcast to the row
// by DPP row_newbcast (every row holds the same 16 values), and w[i] is this
// lane's weight (quads w0..w3).  v_fmac_f32 is fused (one rounding), as the
// chain's definition requires; the leading s_nop covers the wait states a DPP
// read needs after a VALU write of its source.
#define RFMA1(I, W) "v_fmac_f32_dpp %0, %1, " W " row_newbcast:" #I " row_mask:0xf bank_mask:0xf\n\t"
__device__ __forceinline__ void router_fma16_1(float& acc0, float xa, const f4v& w0, const f4v& w1,
                                               const f4v& w2, const f4v& w3) {
  asm volatile("s_nop 1\n\t"
      RFMA1(0, "%2") RFMA1(1, "%3") RFMA1(2, "%4") RFMA1(3, "%5")
      RFMA1(4, "%6") RFMA1(5, "%7") RFMA1(6, "%8") RFMA1(7, "%9")
      RFMA1(8, "%10") RFMA1(9, "%11") RFMA1(10, "%12") RFMA1(11, "%13")
      RFMA1(12, "%14") RFMA1(13, "%15") RFMA1(14, "%16") RFMA1(15, "%17")
      : "+v"(acc0)
      : "v"(xa), "v"(w0.x), "v"(w0.y), "v"(w0.z), "v"(w0.w), "v"(w1.x), "v"(w1.y),
        "v"(w1.z), "v"(w1.w), "v"(w2.x), "v"(w2.y), "v"(w2.z), "v"(w2.w), "v"(w3.x), "v"(w3.y),
        "v"(w3.z), "v"(w3.w));
}
#undef RFMA1

// Reductions over all 64 lanes of a wavefront (every lane active), without
// the LDS crossbar: four DPP steps inside each 16-lane row (swap neighbours,
// swap pairs, mirror the halves of 8, mirror the halves of 16) leave the
// row's result in all of its lanes, then the four rows' results are read
// with v_readlane and combined in a fixed order.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp64(unsigned long long v) {
  const uint32_t lo = dpp32<CTRL>((uint32_t)v), hi = dpp32<CTRL>((uint32_t)(v >> 32));
  return ((unsigned long long)hi << 32) | lo;
}
__device__ __forceinline__ unsigned long long umax64(unsigned long long a, unsigned long long b) {
  return a > b ? a : b;
}
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
  v = umax64(v, dpp64<0xB1>(v));   // quad_perm [1,0,3,2]
  v = umax64(v, dpp64<0x4E>(v));   // quad_perm [2,3,0,1]
  v = umax64(v, dpp64<0x141>(v));  // row_half_mirror
  v = umax64(v, dpp64<0x140>(v));  // row_mirror
  unsigned long long r = 0ull;
#pragma unroll
  for (int row = 0; row < 4; ++row) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 16 * row);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 16 * row);
    r = umax64(r, ((unsigned long long)hi << 32) | lo);
  }
  return r;
}
__device__ __forceinline__ float wave_sum_rows(float v) {
  v += __uint_as_float(dpp32<0xB1>(__float_as_uint(v)));
  v += __uint_as_float(dpp32<0x4E>(__float_as_uint(v)));
  v += __uint_as_float(dpp32<0x141>(__float_as_uint(v)));
  v += __uint_as_float(dpp32<0x140>(__float_as_uint(v)));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// Routing of one tile of ROUTE_TILE tokens, TPT threads per token (threads
// tid < ROUTE_TILE * TPT of the workgroup; every thread of the workgroup
// calls this, since it meets workgroup barriers; both the fused router and
// the routing launch for E > 64 give each token a wavefront).  The tile's logits
// l[token][e] are in LDS.  Top-k by the contract's order (logit descending,
// id ascending): each expert's 64-bit key orders exactly that way and is
// unique, the token's TPT threads hold its keys in registers (expert
// g + TPT c in thread g, NKEY >= E/TPT of them), and slot r takes the largest
// key left after r rounds of a maximum over the TPT threads, its owner
// clearing it.  Then
// softmax over all E, optional renormalisation, and the per-expert rank of
// each (token, slot) pair among the tile's pairs in (token, slot) order, with
// the tile's histogram, for the bucketing kernel.
struct RouteLds {
  float l[ROUTE_TILE][MAX_EXPERTS];
  int ids[ROUTE_TILE * MAX_TOPK];
  float val[ROUTE_TILE][MAX_TOPK];
  int cnt[MAX_EXPERTS];
};

template <int NKEY, int TPT>
__device__ __forceinline__ void route_tile(RouteLds& R, int tile, int t0, int nt, int E, int k, int norm, int tid,
                           int nthreads, int32_t* __restrict__ ids, float* __restrict__ wout,
                           int32_t* __restrict__ rank, int32_t* __restrict__ hist) {
  static_assert(TPT == 16 || TPT == 64, "a token's threads stay inside one wavefront");
  for (int e = tid; e < E; e += nthreads) R.cnt[e] = 0;
  __syncthreads();  // the caller's logit writes are visible to every thread
  // thread (token tl = tid / TPT, lane g = tid % TPT of the token) owns experts g + TPT c
  const int tl = tid / TPT, g = tid % TPT;
  const bool mine = tid < ROUTE_TILE * TPT;
  if (mine) {
    // slots >= k and absent tokens keep -1 (the same wavefront's later
    // stores below land after this one)
    if (g < MAX_TOPK) R.ids[tl * MAX_TOPK + g] = -1;
    unsigned long long key[NKEY];
#pragma unroll
    for (int c = 0; c < NKEY; ++c) {
      const int e = g + TPT * c;
      key[c] = (e < E) ? topk_key(R.l[tl][e], e) : 0ull;  // 0: below every real key
    }
    for (int r = 0; r < k; ++r) {
      unsigned long long m = 0ull;
#pragma unroll
      for (int c = 0; c < NKEY; ++c) m = key[c] > m ? key[c] : m;
      if constexpr (TPT == 64) {
        m = wave_max_u64(m);
      } else {
#pragma unroll
        for (int off = TPT / 2; off > 0; off >>= 1) {
          const unsigned long long o = __shfl_xor(m, off, TPT);
          m = o > m ? o : m;
        }
      }
#pragma unroll
      for (int c = 0; c < NKEY; ++c) key[c] = key[c] == m ? 0ull : key[c];
      if (g == 0 && tl < nt) {
        const int e = (int)~(uint32_t)m;
        R.ids[tl * MAX_TOPK + r] = e;
        R.val[tl][r] = R.l[tl][e];
      }
    }
  }
  __syncthreads();

  if (mine) {
    // softmax over all E (the TPT threads of a token share the sum), weights of the k slots
    const float m = R.val[tl][0];
    float part = 0.0f;
    for (int e = g; e < E; e += TPT) part += expf(R.l[tl][e] - m);
    if constexpr (TPT == 64) {
      part = wave_sum_rows(part);
    } else {
#pragma unroll
      for (int off = TPT / 2; off > 0; off >>= 1) part += __shfl_xor(part, off, TPT);
    }
    float p = (g < k) ? expf(R.val[tl][min(g, k - 1)] - m) / part : 0.0f;
    if (norm) {
      float sum = p;
      if constexpr (TPT == 64) {
        sum = wave_sum_rows(sum);
      } else {
#pragma unroll
        for (int off = TPT / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off, TPT);
      }
      p = p / sum;
    }
    if (tl < nt && g < k) {
      ids[(size_t)(t0 + tl) * k + g] = R.ids[tl * MAX_TOPK + g];
      wout[(size_t)(t0 + tl) * k + g] = p;
    }
  }

  // rank of pair q = (token, slot) among the tile's earlier pairs of the same expert
  const int np = nt * k;
  if (tid < np) {
    const int q = tid;
    const int e = R.ids[(q / k) * MAX_TOPK + q % k];
    int r = 0, later = 0;
    // pairs of earlier tokens (all their k slots), then this token's earlier
    // slots; the ids of two tokens are read per pass, all reads issued before
    // the compares
    for (int t2 = 0; t2 < nt; t2 += 2) {
      // unconditional reads (inside R.ids: t2 + 1 < ROUTE_TILE), masked below
      int4 v[2][MAX_TOPK / 4];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int c4 = 0; c4 < MAX_TOPK / 4; ++c4)
          v[h][c4] = reinterpret_cast<const int4*>(&R.ids[(t2 + h) * MAX_TOPK])[c4];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int c4 = 0; c4 < MAX_TOPK / 4; ++c4) {
          const int ev[4] = {v[h][c4].x, v[h][c4].y, v[h][c4].z, v[h][c4].w};
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            // slots past k and absent tokens hold -1; the order tests are
            // sign bits of differences (no mask operations)
            const int q2 = (t2 + h) * k + 4 * c4 + u;
            const int before = (int)((uint32_t)(q2 - q) >> 31), after = (int)((uint32_t)(q - q2) >> 31);
            const bool same = ev[u] == e;
            r += same ? before : 0;
            later |= same ? after : 0;
          }
        }
    }
    rank[(size_t)(t0 + q / k) * k + q % k] = r;
    if (!later) R.cnt[e] = r + 1;
  }
  __syncthreads();
  for (int e = tid; e < E; e += nthreads) hist[(size_t)tile * E + e] = R.cnt[e];
}

// Router logits for RW tokens x 64 experts per workgroup (lane = expert, one
// token per wavefront, two wavefronts per SIMD).  Each logit is summed in
// fp32 in blocks of 64 j: a fused multiply-add chain over ascending j from +0
// per block, the block sums added in ascending order to a total from +0, then
// + bias (a separate fp32 add); this order is the contract that makes top-k
// ids reproducible bit for bit.
//
// The chains are latency- and operand-bound (one per lane across the whole
// chip at OLMoE sizes), so every operand takes the cheapest path, and two
// wavefronts share each SIMD so that one's LDS reads overlap the other's
// chain.  Per chunk of 64 j the transposed router slab (64 experts x 64 j,
// 16 KiB) and the workgroup's 8 token rows (2 KiB) are copied into a ring of
// LDS buffers RPF chunks ahead.  Per 16 j a lane reads its expert's 16
// weights (4 x 16 B) and one value of its wavefront's token row (lane i of
// every 16-lane row reads column i), and the token value of each step
// reaches all lanes through a DPP row broadcast inside the FMA.  The reads of
// each 16 j are issued three 16-j steps before they are used.  Only the d/16
// sub-chunks inside d are visited (d % 32 == 0), so no padding term enters a
// chain.  (Measured: two wavefronts of one token each run the launch 14 %
// faster than one wavefront per SIMD holding two tokens' chains, although
// they read the slab from LDS twice as often.)
//
// FUSE (E <= 64, so a workgroup holds every logit of its ROUTE_TILE tokens):
// the logits stay in LDS and the workgroup routes its tile (route_tile), with
// no logits in global memory and no separate routing launch.
template <bool FUSE, int RNB>
__global__ __launch_bounds__(512) void router_kernel(
    const float* __restrict__ x, int n, int d, const float* __restrict__ wt,
    const float* __restrict__ bias, int E, int E64, float* __restrict__ logits, int k, int norm,
    int32_t* __restrict__ ids, float* __restrict__ wout, int32_t* __restrict__ rank,
    int32_t* __restrict__ hist) {
  constexpr int RPF = RNB - 1;  // chunks copied ahead
  __shared__ __attribute__((aligned(1024))) char ring[RNB * R_BUF];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int eg = blockIdx.y;
  const int tw = blockIdx.x * RW * RT + wave * RT;  // this wavefront's token
  const int C = (d + RJC - 1) / RJC, NQ = d / 4;
  const uint32_t lbase = (uint32_t)(uintptr_t)(lds_char*)ring;
  const float* xr0 = x + (size_t)min(tw, n - 1) * d;

  // Wavefront w copies quads 2w, 2w+1 of the slab (1 KiB each: the 64
  // experts' 4 j; quads past d re-read the last one) and its own token row
  // (columns past d re-read column d-1).
  auto issue = [&](int c) {
    const uint32_t buf = lbase + (uint32_t)((c % RNB) * R_BUF);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int jq = min(c * RJQ + 2 * wave + i, NQ - 1);
      rdma16(wt + ((size_t)jq * E64 + eg * 64) * 4, lane * 16, buf + (2 * wave + i) * 1024);
    }
    const uint32_t xo = (uint32_t)min(c * RJC + lane, d - 1) * 4;
    rdma4(xr0, xo, buf + R_WB + (RT * wave) * (RJC * 4));
  };
  const int np = min(RPF, C);
  for (int c = 0; c < np; ++c) issue(c);

  // Wait until chunk c is copied for every wavefront, given how many chunks
  // this wavefront has issued after it (vector loads complete in order).
  static_assert(RPF <= 7 && RPF * RDMA <= 63, "vmcnt counts at most 63 copies");
  auto wait_chunk = [&](int newer) {
    switch (newer) {
      case 0: rwait_vm<0>(); break;
      case 1: rwait_vm<RDMA>(); break;
      case 2: rwait_vm<2 * RDMA>(); break;
      case 3: rwait_vm<3 * RDMA>(); break;
      case 4: rwait_vm<4 * RDMA>(); break;
      case 5: rwait_vm<5 * RDMA>(); break;
      default: rwait_vm<6 * RDMA>(); break;
    }
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // operands of 16-j sub-chunks, a ring of 4 (read 3 sub-chunks ahead)
  f4v w[4][4];
  float xa[4];
  auto load_sub = [&](int sub, int b) {
    const int c = sub >> 2, q0 = (sub & 3) * 4;
    const char* buf = ring + (c % RNB) * R_BUF;
#pragma unroll
    for (int q = 0; q < 4; ++q) w[b][q] = *reinterpret_cast<const f4v*>(buf + (q0 + q) * 1024 + lane * 16);
    const float* xrow = reinterpret_cast<const float*>(buf + R_WB) + (RT * wave) * RJC + q0 * 4 + (lane & 15);
    xa[b] = xrow[0];
  };
  // The logit's blocks of 64 j are the chunks: acc0 chains one chunk from +0,
  // total adds the finished chunks in order.
  float acc0 = 0.0f, total = 0.0f;
  // One full chunk (4 sub-chunks of 16 j) per iteration, then the trailing
  // half chunk when d % 64 == 32.  The reads of sub-chunk s+3 are issued
  // before sub-chunk s is computed, unconditionally (past the last sub-chunk
  // they read stale LDS and are discarded).  At the first sub-chunk of chunk c
  // chunk c+1 is waited for and published (its sub-chunk 0 is read from the
  // next step on); every wavefront has then read all of chunk c-1, whose
  // buffer takes chunk c+RPF.
  const int CF = d / RJC;
  // A wavefront whose tokens are all past n (small batches) computes nothing
  // but still does its share of the copies and meets every barrier.
  const bool busy = tw < n;  // wavefront-uniform
  wait_chunk(np - 1);  // chunks 1..np-1 were issued after chunk 0
  if (busy) {
    load_sub(0, 0);
    load_sub(1, 1);
    load_sub(2, 2);
  }
  for (int c = 0; c < CF; ++c) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (q == 0 && c + 1 < C) {
        // issued so far: chunks 0 .. min(c+RPF-1, C-1); newer than c+1: the rest
        wait_chunk(min(RPF - 2, C - c - 2));
        if (c + RPF < C) issue(c + RPF);
      }
      if (busy) {
        load_sub(4 * c + q + 3, (q + 3) & 3);
        router_fma16_1(acc0, xa[q], w[q][0], w[q][1], w[q][2], w[q][3]);
      }
    }
    total += acc0;
    acc0 = 0.0f;
  }
  if (busy && CF < C) {  // 32 trailing j (the last block): sub-chunks 4 CF and 4 CF + 1 (already requested)
    router_fma16_1(acc0, xa[0], w[0][0], w[0][1], w[0][2], w[0][3]);
    router_fma16_1(acc0, xa[1], w[1][0], w[1][1], w[1][2], w[1][3]);
    total += acc0;
  }
  const int e = eg * 64 + lane;
  if constexpr (FUSE) {
    static_assert(RW * RT == ROUTE_TILE, "a router workgroup covers one routing tile");
    __shared__ __attribute__((aligned(16))) RouteLds R;
    const int tl = wave * RT;
    if (e < E) {
      const float bb = bias ? bias[e] : 0.0f;
      R.l[tl][e] = bias ? total + bb : total;
    }
    const int t0 = blockIdx.x * ROUTE_TILE;
    route_tile<1, 64>(R, blockIdx.x, t0, min(ROUTE_TILE, n - t0), E, k, norm, threadIdx.x, 512, ids, wout,
               rank, hist);
  } else {
    if (e < E) {
      const float bb = bias ? bias[e] : 0.0f;
      if (tw < n) logits[(size_t)tw * E + e] = bias ? total + bb : total;
    }
  }
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// The tile's logits from global memory into LDS.
// (ROUTE_WIDE_THREADS threads; every load is issued before the first LDS
// store, one memory round trip: the index is clamped into the tile's logits
// and the surplus masked)
constexpr int ROUTE_WIDE_THREADS = ROUTE_TILE * 64;  // one wavefront per token
__device__ __forceinline__ void route_load_logits(RouteLds& R, const float* __restrict__ logits, int t0, int nt, int E,
                                  int tid) {
  constexpr int PER = ROUTE_TILE * MAX_EXPERTS / ROUTE_WIDE_THREADS;
  const int tot = nt * E;
  float v[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) v[u] = logits[(size_t)t0 * E + min(tid + u * ROUTE_WIDE_THREADS, tot - 1)];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int i = tid + u * ROUTE_WIDE_THREADS;
    if (i < ROUTE_TILE * E) {
      const int tl = i / E, e = i - tl * E;
      R.l[tl][e] = (i < tot) ? v[u] : 0.0f;
    }
  }
}

// Routing as its own kernel (E > 64: a router workgroup holds only a 64-expert
// slice of its tokens' logits).  One workgroup per ROUTE_TILE tokens.
__global__ __launch_bounds__(ROUTE_WIDE_THREADS) void route_kernel(
    const float* __restrict__ logits, int n, int E, int k, int norm, int32_t* __restrict__ ids,
    float* __restrict__ wout, int32_t* __restrict__ rank, int32_t* __restrict__ hist) {
  __shared__ __attribute__((aligned(16))) RouteLds R;
  const int t0 = blockIdx.x * ROUTE_TILE;
  const int nt = min(ROUTE_TILE, n - t0);
  route_load_logits(R, logits, t0, nt, E, threadIdx.x);
  route_tile<MAX_EXPERTS / 64, 64>(R, blockIdx.x, t0, nt, E, k, norm, threadIdx.x, ROUTE_WIDE_THREADS, ids, wout, rank,
                                   hist);
}

// ---------------------------------------------------------------- decode
// Decode router (1 <= N <= 8).  The same logits as router_kernel (fp32;
// blocks of 64 j, each chained by fused multiply-adds over ascending j from
// +0; block sums added in ascending order, then the bias), but with too few
// tokens to share the router matrix among many of them, so the blocks of a
// logit run in parallel: one lane per (expert, block), and the block sums
// are added in order afterwards.  A workgroup covers DR_E experts and, per
// pass, DR_NBP blocks (2048 j): lane (e, b) reads its block's 16 weight quads
// straight from the transposed matrix [d/4][E64][4] into registers (8
// experts' quads of one j are 128 contiguous bytes) and its tokens' values
// from LDS, where the workgroup stages the pass's N x 2048 slice of x.  The
// block sums meet in LDS and lane (e, t) adds them in block order.  The
// workgroups past the router ones quantise one token row each (the same
// pieces, decisions and shared-gate order as the prefill quantiser in the
// bucketing launch), writing the token-major codes the decode matvecs read.
constexpr int DR_E = 8;                       // experts per router workgroup
constexpr int DR_RB = 64;                     // j per block of the logit's sum
constexpr int DR_NBP = 32;                    // blocks per pass: DR_E x DR_NBP = 256 lanes
constexpr int DR_JP = DR_RB * DR_NBP;         // j per pass
constexpr int DR_XBLK = DR_RB + 4;            // staged floats per block (+4: the 8 blocks a
                                              // wavefront reads at once start in different banks)
constexpr int DR_XTOK = DR_NBP * DR_XBLK;     // staged floats per token and pass
static_assert(DR_E * DR_NBP == 256, "one (expert, block) per lane");

// Quantise token row xr (one wavefront): pass j0 covers values [1024 j0', +1024),
// lane l the 16 values from 16 l; codes/scales to xq_row/xs_row up to d_pad
// (zero past d); with shg the shared-gate dot product in the prefill order.
__device__ __forceinline__ void decode_quantize_row(const float* __restrict__ xr, int d, int d_pad,
                                                    const float* __restrict__ shg, float* __restrict__ gs_t,
                                                    int8_t* __restrict__ xq_row,
                                                    uint16_t* __restrict__ xs_row, int lane) {
  float gacc = 0.0f;
  for (int c00 = 0; c00 < d_pad; c00 += 1024) {
    const int c0 = c00 + lane * 16;
    const bool valid = c0 < d;  // d % 32 == 0: a piece is all valid or all padding
    const float* src = xr + (valid ? c0 : 0);
    f4v a4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a4[i] = *reinterpret_cast<const f4v*>(src + 4 * i);
    float v[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[4 * i] = valid ? a4[i].x : 0.0f;
      v[4 * i + 1] = valid ? a4[i].y : 0.0f;
      v[4 * i + 2] = valid ? a4[i].z : 0.0f;
      v[4 * i + 3] = valid ? a4[i].w : 0.0f;
    }
    uint32_t pk[4];
    uint16_t s16;
    quant_half_block16(v, pk, s16);
    if (c0 < d_pad) {
      *reinterpret_cast<uint4*>(xq_row + c0) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      if ((lane & 1) == 0) xs_row[c0 / QB] = s16;
    }
    if (shg && valid) {
#pragma unroll
      for (int i = 0; i < 16; ++i) gacc = __builtin_fmaf(v[i], shg[c0 + i], gacc);
    }
  }
  if (shg) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) gacc += __shfl_xor(gacc, off, 64);
    if (lane == 0) *gs_t = 1.0f / (1.0f + expf(-gacc));
  }
}

template <int NT>
__global__ __launch_bounds__(256, 1) void decode_router_kernel(
    const float* __restrict__ x, int n, int d, int d_pad, const float* __restrict__ wt,
    const float* __restrict__ bias, int E, int E64, int n_rwg, float* __restrict__ logits,
    const float* __restrict__ shg, float* __restrict__ gs, int8_t* __restrict__ xq,
    uint16_t* __restrict__ xs) {
  __shared__ __attribute__((aligned(16))) float xl[NT * DR_XTOK];
  __shared__ __attribute__((aligned(16))) float part[NT][DR_E][DR_NBP + 4];  // +4: bank offset per expert
  const int tid = threadIdx.x, lane = tid & 63;
  if ((int)blockIdx.x >= n_rwg) {
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int t = (int)blockIdx.x - n_rwg;
    if (wave == 0 && t < n)
      decode_quantize_row(x + (size_t)t * d, d, d_pad, shg, gs + t, xq + (size_t)t * d_pad,
                          xs + (size_t)t * (d_pad / QB), lane);
    return;
  }
  const int el = tid % DR_E, bl = tid / DR_E;
  const int e = DR_E * (int)blockIdx.x + el;  // < E64: the matrix holds zero rows past E
  // lane (el, t) of the first DR_E * NT lanes adds the block sums of (e, t)
  const int se = tid % DR_E, st = tid / DR_E;
  float total = 0.0f;
  for (int j0 = 0; j0 < d; j0 += DR_JP) {
    // this pass's token values: [t][block][DR_XBLK], quads past d skipped
    constexpr int XQ = NT * DR_JP / 4;  // quads to stage
    f4v xv[(XQ + 255) / 256];
#pragma unroll
    for (int u = 0; u < (XQ + 255) / 256; ++u) {
      const int i = tid + 256 * u, t = i / (DR_JP / 4), jq = i % (DR_JP / 4);
      if (i < XQ && j0 + 4 * jq < d)
        xv[u] = *reinterpret_cast<const f4v*>(x + (size_t)t * d + j0 + 4 * jq);
    }
    // this lane's weights: quads q of block bl (16 per full block; d % 32 == 0,
    // so a block past d's last full one has 8 or none)
    const int jb = j0 + DR_RB * bl;
    const int nq = max(0, min(DR_RB, d - jb)) / 4;
    f4v w[DR_RB / 4];
#pragma unroll
    for (int q = 0; q < DR_RB / 4; ++q)
      if (q < nq) w[q] = *reinterpret_cast<const f4v*>(wt + ((size_t)(jb / 4 + q) * E64 + e) * 4);
    if (j0 > 0) __syncthreads();  // every lane is done with the previous pass's values
#pragma unroll
    for (int u = 0; u < (XQ + 255) / 256; ++u) {
      const int i = tid + 256 * u, t = i / (DR_JP / 4), jq = i % (DR_JP / 4);
      if (i < XQ && j0 + 4 * jq < d)
        *reinterpret_cast<f4v*>(xl + t * DR_XTOK + (jq / 16) * DR_XBLK + 4 * (jq % 16)) = xv[u];
    }
    __syncthreads();
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = 0.0f;
    const float* xb = xl + bl * DR_XBLK;
    auto quads = [&](int q0, int q1) {
#pragma unroll
      for (int q = q0; q < q1; ++q) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const f4v v = *reinterpret_cast<const f4v*>(xb + t * DR_XTOK + 4 * q);
          acc[t] = __builtin_fmaf(v.x, w[q].x, acc[t]);
          acc[t] = __builtin_fmaf(v.y, w[q].y, acc[t]);
          acc[t] = __builtin_fmaf(v.z, w[q].z, acc[t]);
          acc[t] = __builtin_fmaf(v.w, w[q].w, acc[t]);
        }
      }
    };
    if (nq > 0) quads(0, DR_RB / 8);
    if (nq == DR_RB / 4) quads(DR_RB / 8, DR_RB / 4);
#pragma unroll
    for (int t = 0; t < NT; ++t) part[t][el][bl] = acc[t];
    __syncthreads();
    if (st < NT) {
      // all of the pass's block sums read at once (past nb: stale, unused)
      const int nb = min(DR_NBP, (d - j0 + DR_RB - 1) / DR_RB);
      f4v pv[DR_NBP / 4];
#pragma unroll
      for (int b4 = 0; b4 < DR_NBP / 4; ++b4) pv[b4] = *reinterpret_cast<const f4v*>(&part[st][se][4 * b4]);
#pragma unroll
      for (int b = 0; b < DR_NBP; ++b)
        if (b < nb) total += pv[b / 4][b % 4];
    }
  }
  const int eo = DR_E * (int)blockIdx.x + se;
  if (st < NT && st < n && eo < E) logits[(size_t)st * E + eo] = bias ? total + bias[eo] : total;
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
                         int E64, float* logits, int n_cu, hipStream_t s) {
  dim3 grid((unsigned)((n + RW * RT - 1) / (RW * RT)), (unsigned)(E64 / 64));
  if ((long)grid.x * grid.y > n_cu)
    router_kernel<false, RNB_SHALLOW><<<grid, 512, 0, s>>>(x, n, d, wt, bias, E, E64, logits, 0, 0, nullptr,
                                                           nullptr, nullptr, nullptr);
  else
    router_kernel<false, RNB_DEEP><<<grid, 512, 0, s>>>(x, n, d, wt, bias, E, E64, logits, 0, 0, nullptr,
                                                        nullptr, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_router_route(const float* x, int n, int d, const float* wt, const float* bias,
                               int E, int k, int norm, int32_t* ids, float* w, int32_t* rank,
                               int32_t* hist, int n_cu, hipStream_t s) {
  if (E > 64) return hipErrorInvalidValue;
  dim3 grid((unsigned)((n + ROUTE_TILE - 1) / ROUTE_TILE), 1);
  if ((long)grid.x > n_cu)
    router_kernel<true, RNB_SHALLOW><<<grid, 512, 0, s>>>(x, n, d, wt, bias, E, 64, nullptr, k, norm, ids, w,
                                                          rank, hist);
  else
    router_kernel<true, RNB_DEEP><<<grid, 512, 0, s>>>(x, n, d, wt, bias, E, 64, nullptr, k, norm, ids, w,
                                                       rank, hist);
  return hipGetLastError();
}

hipError_t launch_route(const float* logits, int n, int E, int k, int norm, int32_t* ids, float* w,
                        int32_t* rank, int32_t* hist, hipStream_t s) {
  const int tiles = (n + ROUTE_TILE - 1) / ROUTE_TILE;
  route_kernel<<<tiles, ROUTE_WIDE_THREADS, 0, s>>>(logits, n, E, k, norm, ids, w, rank, hist);
  return hipGetLastError();
}

hipError_t launch_decode_router(const float* x, int n, int d, int d_pad, const float* wt,
                                const float* bias, int E, int E64, float* logits,
                                const float* sh_gate_vec, float* gs, int8_t* dxq, uint16_t* dxs,
                                hipStream_t s) {
  if (n < 1 || n > DECODE_MAX_TOKENS) return hipErrorInvalidValue;
  const int n_rwg = (E + DR_E - 1) / DR_E;
#define DR_LAUNCH(NT)                                                                             \
  case NT:                                                                                         \
    decode_router_kernel<NT><<<n_rwg + n, 256, 0, s>>>(x, n, d, d_pad, wt, bias, E, E64, n_rwg, logits, \
                                                       sh_gate_vec, gs, dxq, dxs);                 \
    break;
  static_assert(DECODE_MAX_TOKENS == 8, "one instantiation per batch size");
  switch (n) {
    DR_LAUNCH(1) DR_LAUNCH(2) DR_LAUNCH(3) DR_LAUNCH(4) DR_LAUNCH(5) DR_LAUNCH(6) DR_LAUNCH(7) DR_LAUNCH(8)
  }
#undef DR_LAUNCH
  return hipGetLastError();
}

hipError_t launch_quantize(const float* v, int64_t n_values, int8_t* q, uint16_t* scales,
                           hipStream_t s) {
  const int64_t blocks = (n_values + 255) / 256;
  quantize_kernel<<<(unsigned)blocks, 256, 0, s>>>(v, n_values, q, scales);
  return hipGetLastError();
}

}  // namespace moe
