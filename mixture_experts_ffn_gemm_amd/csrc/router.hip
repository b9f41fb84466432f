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
#include "route_util.h"
#include "internal.h"

namespace moe {
namespace {

typedef float f4v __attribute__((ext_vector_type(4)));

constexpr int RB = 64;            // j per block of a logit's sum
constexpr int RWV = 8;            // prefill router: wavefronts per workgroup
constexpr int RJR = RB * RWV;     // j per round (one block per wavefront)
static_assert(RWV == ROUTE_TILE, "thread (token, expert) of the block sums is (wavefront, lane)");

// 16 steps of two fp32 fused multiply-add chains: for i = 0..15,
//   acc0 = fma(x0[i], w[i], acc0),  acc1 = fma(x1[i], w[i], acc1),
// where xN[i] is lane i of this lane's 16-lane row of xN, broadcast to the row
// by DPP row_newbcast (every row holds the same 16 values), and w[i] is this
// lane's weight (quads w0..w3).  v_fmac_f32 is fused (one rounding), as the
// block chain's definition requires; the two chains alternate so that each
// step's dependency is two instructions old, and the leading s_nop covers the
// wait states a DPP read needs after a VALU write of its source.
#define RFMA2(I, W)                                                                  \
  "v_fmac_f32_dpp %0, %2, " W " row_newbcast:" #I " row_mask:0xf bank_mask:0xf\n\t" \
  "v_fmac_f32_dpp %1, %3, " W " row_newbcast:" #I " row_mask:0xf bank_mask:0xf\n\t"
__device__ __forceinline__ void router_fma16_2(float& acc0, float& acc1, float x0, float x1, const f4v& w0,
                                               const f4v& w1, const f4v& w2, const f4v& w3) {
  asm volatile("s_nop 1\n\t"
      RFMA2(0, "%4") RFMA2(1, "%5") RFMA2(2, "%6") RFMA2(3, "%7")
      RFMA2(4, "%8") RFMA2(5, "%9") RFMA2(6, "%10") RFMA2(7, "%11")
      RFMA2(8, "%12") RFMA2(9, "%13") RFMA2(10, "%14") RFMA2(11, "%15")
      RFMA2(12, "%16") RFMA2(13, "%17") RFMA2(14, "%18") RFMA2(15, "%19")
      : "+v"(acc0), "+v"(acc1)
      : "v"(x0), "v"(x1), "v"(w0.x), "v"(w0.y), "v"(w0.z), "v"(w0.w), "v"(w1.x), "v"(w1.y),
        "v"(w1.z), "v"(w1.w), "v"(w2.x), "v"(w2.y), "v"(w2.z), "v"(w2.w), "v"(w3.x), "v"(w3.y),
        "v"(w3.z), "v"(w3.w));
}
#undef RFMA2
#define RFMA1(I, W) "v_fmac_f32_dpp %0, %1, " W " row_newbcast:" #I " row_mask:0xf bank_mask:0xf\n\t"
// One chain of router_fma16_2's form (a batch with an odd token count).
__device__ __forceinline__ void router_fma16_1(float& acc0, float x0, const f4v& w0, const f4v& w1, const f4v& w2,
                                               const f4v& w3) {
  asm volatile("s_nop 1\n\t"
      RFMA1(0, "%2") RFMA1(1, "%3") RFMA1(2, "%4") RFMA1(3, "%5")
      RFMA1(4, "%6") RFMA1(5, "%7") RFMA1(6, "%8") RFMA1(7, "%9")
      RFMA1(8, "%10") RFMA1(9, "%11") RFMA1(10, "%12") RFMA1(11, "%13")
      RFMA1(12, "%14") RFMA1(13, "%15") RFMA1(14, "%16") RFMA1(15, "%17")
      : "+v"(acc0)
      : "v"(x0), "v"(w0.x), "v"(w0.y), "v"(w0.z), "v"(w0.w), "v"(w1.x), "v"(w1.y),
        "v"(w1.z), "v"(w1.w), "v"(w2.x), "v"(w2.y), "v"(w2.z), "v"(w2.w), "v"(w3.x), "v"(w3.y),
        "v"(w3.z), "v"(w3.w));
}
#undef RFMA1

// Sum over all 64 lanes of a wavefront (every lane active), without the LDS
// crossbar: four DPP steps inside each 16-lane row (swap neighbours, swap
// pairs, mirror the halves of 8, mirror the halves of 16) leave the row's sum
// in all of its lanes, then the four rows' sums are read with v_readlane and
// added in a fixed order.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
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

// Routing of one tile of ROUTE_TILE tokens, one wavefront per token (threads
// tid < ROUTE_TILE * 64 of the workgroup; every thread of the workgroup calls
// this, since it meets workgroup barriers).  The tile's logits l[token][e] are
// in LDS.  Top-k by the contract's order (logit descending, id ascending): each
// expert's 64-bit key orders exactly that way and is unique; lane g holds the
// keys of experts g + 64c, and slot r takes the largest key left after r
// rounds of a wavefront maximum, its owner clearing it.  The maximum is
// uniform, so lane r keeps slot r's expert and logit (decoded from the key).
// With one key per lane (E <= 64) a single pass ranks every key instead
// (wave_key_rank): the rank of a key is its slot.
// Then softmax over all E, optional renormalisation, and, for the bucketing
// kernel, the per-expert rank of each (token, slot) pair among the tile's
// pairs in (token, slot) order and the tile's histogram.  A token's k experts
// are distinct, so a pair's rank is the number of earlier tokens of the tile
// that picked the same expert: both come from per-token ballots of the picked
// experts.
struct RouteLds {
  float l[ROUTE_TILE][MAX_EXPERTS];
  unsigned long long pick[ROUTE_TILE][MAX_EXPERTS / 64];  // bit g of [t][c]: token t picked expert g + 64c
  __attribute__((aligned(16))) unsigned long long kl[ROUTE_TILE][64];  // E <= 64: each token's keys (wave_key_rank)
  int sel_id[ROUTE_TILE][MAX_TOPK];                       // E <= 64: slot s's expert and logit
  float sel_v[ROUTE_TILE][MAX_TOPK];
};

// The logit a key was made from (-0 comes back as +0).
__device__ __forceinline__ float key_logit(unsigned long long key) {
  const uint32_t ord = (uint32_t)(key >> 32);
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord);
}

template <int NKEY>
__device__ __forceinline__ void route_tile(RouteLds& R, int tile, int t0, int nt, int E, int k, int norm, int tid,
                                           int32_t* __restrict__ ids, float* __restrict__ wout,
                                           int32_t* __restrict__ rank, int32_t* __restrict__ hist) {
  __syncthreads();  // the caller's logit writes are visible to every thread
  const int tl = tid >> 6, g = tid & 63;
  const bool mine = tid < ROUTE_TILE * 64;  // wavefront-uniform
  int slot[NKEY];
  if (mine) {
    unsigned long long key[NKEY];
#pragma unroll
    for (int c = 0; c < NKEY; ++c) {
      const int e = g + 64 * c;
      key[c] = (e < E) ? topk_key(R.l[tl][e], e) : 0ull;  // 0: below every real key
      slot[c] = -1;
    }
    int my_id = 0;
    float my_val = 0.0f;
    if constexpr (NKEY == 1) {
      // one key per lane: its rank is its slot (keys are distinct); slot r's
      // expert and logit reach lane r through LDS
      const int rk = wave_key_rank(key[0], R.kl[tl], g);
      if (g < E && rk < k) {
        slot[0] = rk;
        R.sel_id[tl][rk] = g;
        R.sel_v[tl][rk] = key_logit(key[0]);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (g < k) {
        my_id = R.sel_id[tl][g];
        my_val = R.sel_v[tl][g];
      }
    } else {
      for (int r = 0; r < k; ++r) {
        unsigned long long m = 0ull;
#pragma unroll
        for (int c = 0; c < NKEY; ++c) m = key[c] > m ? key[c] : m;
        m = wave_max_key(m);
#pragma unroll
        for (int c = 0; c < NKEY; ++c) {
          const bool hit = key[c] == m;
          slot[c] = hit ? r : slot[c];
          key[c] = hit ? 0ull : key[c];
        }
        if (g == r) {
          my_id = (int)~(uint32_t)m;
          my_val = key_logit(m);
        }
      }
    }
    // softmax over all E, weights of the k slots (lane s: slot s)
    const float m0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_val), 0));
    float part = 0.0f;
#pragma unroll
    for (int c = 0; c < NKEY; ++c) {
      const int e = g + 64 * c;
      if (e < E) part += expf(R.l[tl][e] - m0);
    }
    part = wave_sum_rows(part);
    float p = (g < k) ? expf(my_val - m0) / part : 0.0f;
    if (norm) p = p / wave_sum_rows(p);
    if (tl < nt && g < k) {
      ids[(size_t)(t0 + tl) * k + g] = my_id;
      wout[(size_t)(t0 + tl) * k + g] = p;
    }
#pragma unroll
    for (int c = 0; c < NKEY; ++c) {
      const unsigned long long b = __ballot(slot[c] >= 0);
      if (g == 0) R.pick[tl][c] = (tl < nt) ? b : 0ull;  // absent tokens pick nothing
    }
  }
  __syncthreads();
  if (mine) {
#pragma unroll
    for (int c = 0; c < NKEY; ++c) {
      if (tl < nt && slot[c] >= 0) {
        int rk = 0;
#pragma unroll
        for (int t2 = 0; t2 < ROUTE_TILE; ++t2) rk += (t2 < tl) ? (int)((R.pick[t2][c] >> g) & 1ull) : 0;
        rank[(size_t)(t0 + tl) * k + slot[c]] = rk;
      }
      const int e = g + 64 * c;
      if (tl == 0 && e < E) {
        int cnt = 0;
#pragma unroll
        for (int t2 = 0; t2 < ROUTE_TILE; ++t2) cnt += (int)((R.pick[t2][c] >> g) & 1ull);
        hist[(size_t)tile * E + e] = cnt;
      }
    }
  }
}

// Router logits for ROUTE_TILE (8) tokens x 64 experts per workgroup (lane =
// expert).  Each logit is summed in fp32 in blocks of 64 j: a fused
// multiply-add chain over ascending j from +0 per block, the block sums added
// in ascending order to a total from +0, then + bias (a separate fp32 add);
// this order is the contract that makes top-k ids reproducible bit for bit.
//
// The blocks of a logit are independent until they are added, so the work is
// split by block: in round r wavefront w chains block 8r + w for all 8 tokens.
// A lane holds its expert's 64 weights of the block in registers (16 quads
// read straight from the transposed matrix [d/4][E64][4], where the 64
// experts' quads of one j are 1 KiB), so each weight is read once per
// workgroup and used for 8 tokens, and the only LDS traffic is the token
// values: lane i of each 16-lane row reads value i of a 16-j piece, and a DPP
// row broadcast inside the FMA hands each step's value to the row.  The
// round's 8 block sums per (token, expert) meet in LDS, and thread (token w,
// expert lane) adds them to its total in block order.  The token values of
// round r+1 are staged through registers into LDS during round r, and each
// wavefront's weights are requested two rounds ahead.
//
// FUSE (E <= 64, so a workgroup holds every logit of its ROUTE_TILE tokens):
// the logits stay in LDS and the workgroup routes its tile (route_tile), with
// no logits in global memory and no separate routing launch.
// WB: weight buffers per wavefront.  2: round r+2's weights are requested
// during round r (one workgroup per CU); 1: round r+1's after round r is
// computed, at most 128 VGPRs (four wavefronts per SIMD), so that two
// workgroups share a CU and each hides the other's waits (grids with more
// workgroups than CUs).
template <bool FUSE, int WB>
__global__ __launch_bounds__(512, 6 - 2 * WB) void router_kernel(
    const float* __restrict__ x, int n, int d, const float* __restrict__ wt,
    const float* __restrict__ bias, int E, int E64, float* __restrict__ logits, int k, int norm,
    int32_t* __restrict__ ids, float* __restrict__ wout, int32_t* __restrict__ rank,
    int32_t* __restrict__ hist) {
  __shared__ __attribute__((aligned(16))) float xs[2][ROUTE_TILE][RJR];   // token values per round
  __shared__ __attribute__((aligned(16))) float ps[2][ROUTE_TILE][RWV][64];  // block sums per round
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int eg = blockIdx.y;
  const int t0 = blockIdx.x * ROUTE_TILE;
  const int NB = (d + RB - 1) / RB, NR = (NB + RWV - 1) / RWV, NQ = d / 4;
  const float* wcol = wt + (size_t)(eg * 64 + lane) * 4;

  // Round r's token values: thread tid moves quads tid and tid + 512 of the
  // 8 x 128 (tokens past n re-read token n-1, columns past d the last quad).
  auto load_x = [&](int r, f4v (&v)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = tid + 512 * i, t = q >> 7, jq = q & 127;
      const int tc = min(t0 + t, n - 1), j = min(r * RJR + 4 * jq, d - 4);
      v[i] = *reinterpret_cast<const f4v*>(x + (size_t)tc * d + j);
    }
  };
  auto store_x = [&](int bi, const f4v (&v)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = tid + 512 * i, t = q >> 7, jq = q & 127;
      *reinterpret_cast<f4v*>(&xs[bi][t][4 * jq]) = v[i];
    }
  };
  // This wavefront's block of round r: the lane's 16 weight quads (a block
  // past d re-reads the last one, quads past d the last quad; neither is used).
  auto load_w = [&](int r, f4v (&w)[16]) {
    const int b = min(r * RWV + wave, NB - 1);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int jq = min(16 * b + q, NQ - 1);
      w[q] = *reinterpret_cast<const f4v*>(wcol + (size_t)jq * E64 * 4);
    }
  };
  // Round r from buffer bi: the block sums of this wavefront's block for the
  // 8 tokens into ps[bi][t][wave][lane] (0 past the last block).
  auto compute = [&](int r, int bi, const f4v (&w)[16]) {
    const int b = r * RWV + wave;
    float acc[ROUTE_TILE];
#pragma unroll
    for (int t = 0; t < ROUTE_TILE; ++t) acc[t] = 0.0f;
    if (b < NB) {  // wavefront-uniform
      const bool full = d - RB * b >= RB;  // else 32 j (d % 32 == 0): sub-chunks 0 and 1
      const float* xb = &xs[bi][0][RB * wave] + (lane & 15);
      // WB == 2: every token value of the block requested before the first FMA
      // (one LDS latency per round, not one per 16-step piece; past a half
      // block the reads are stale and unused).  WB == 1 (128 VGPRs): per pair.
      constexpr int XR = WB == 2 ? ROUTE_TILE : 2;
      float xr[XR][4];
      auto fetch = [&](int t0x, int nt) {
#pragma unroll
        for (int t = 0; t < nt; ++t)
#pragma unroll
          for (int s = 0; s < 4; ++s) xr[(t0x + t) % XR][s] = xb[(t0x + t) * RJR + 16 * s];
      };
      if constexpr (WB == 2) fetch(0, ROUTE_TILE);
#pragma unroll
      for (int tp = 0; tp < ROUTE_TILE / 2; ++tp) {
        if constexpr (WB == 1) fetch(2 * tp, 2);
#pragma unroll
        for (int s = 0; s < 4; ++s)
          if (s < 2 || full)
            router_fma16_2(acc[2 * tp], acc[2 * tp + 1], xr[(2 * tp) % XR][s], xr[(2 * tp + 1) % XR][s], w[4 * s],
                           w[4 * s + 1], w[4 * s + 2], w[4 * s + 3]);
      }
    }
#pragma unroll
    for (int t = 0; t < ROUTE_TILE; ++t) ps[bi][t][wave][lane] = acc[t];
  };

  // token values are requested two rounds ahead (register sets xA, xB for
  // even and odd rounds), weights per WB
  f4v xA[2], xB[2], wA[16], wB[WB == 2 ? 16 : 1];
  float total = 0.0f;
  // Round 0's operands first and alone (every CU requests them at once, and
  // later requests would share the bandwidth they arrive by); the next
  // rounds' requests follow the barrier and arrive during round 0.
  load_x(0, xA);
  load_w(0, wA);
  store_x(0, xA);
  __syncthreads();
  if (NR > 1) {
    load_x(1, xB);
    if constexpr (WB == 2) load_w(1, wB);
  }
  if (NR > 2) load_x(2, xA);
  // One round: compute it, stage round r+1's values (their buffer was last
  // read in round r-1, before its barrier) and request round r+3's into the
  // freed registers, request the next weights, then (after the barrier) fold
  // the round's block sums into the total in block order.
  auto round = [&](int r, f4v (&w)[16], f4v (&xn)[2]) {
    const int bi = r & 1;
    compute(r, bi, w);
    if (r + 1 < NR) store_x(bi ^ 1, xn);
    if (r + 3 < NR) load_x(r + 3, xn);
    if constexpr (WB == 2) {
      if (r + 2 < NR) load_w(r + 2, w);
    } else {
      if (r + 1 < NR) load_w(r + 1, w);
    }
    __syncthreads();
    const int nb = min(RWV, NB - r * RWV);
#pragma unroll
    for (int bb = 0; bb < RWV; ++bb)
      if (bb < nb) total += ps[bi][wave][bb][lane];
  };
  // unrolled by two so that each register set has a fixed role
  for (int r = 0; r < NR; r += 2) {
    round(r, wA, xB);
    if constexpr (WB == 2) {
      if (r + 1 < NR) round(r + 1, wB, xA);
    } else {
      if (r + 1 < NR) round(r + 1, wA, xA);
    }
  }

  const int e = eg * 64 + lane;
  const int tw = t0 + wave;  // this thread's token
  if constexpr (FUSE) {
    __shared__ __attribute__((aligned(16))) RouteLds R;
    if (e < E) {
      const float bb = bias ? bias[e] : 0.0f;
      R.l[wave][e] = bias ? total + bb : total;
    }
    route_tile<1>(R, blockIdx.x, t0, min(ROUTE_TILE, n - t0), E, k, norm, threadIdx.x, ids, wout, rank, hist);
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
// (zero past d), and to xq_out/xs_out (optional) up to d; with shg the
// shared-gate dot product.  Pieces, decisions and the gate's order are those
// of the prefill quantiser in the bucketing launch, so the results are
// bit-identical.
__device__ __forceinline__ void quantize_row(const float* __restrict__ xr, int d, int d_pad,
                                             const float* __restrict__ shg, float* __restrict__ gs_t,
                                             int8_t* __restrict__ xq_row, uint16_t* __restrict__ xs_row,
                                             int8_t* __restrict__ xq_out, uint16_t* __restrict__ xs_out,
                                             int lane) {
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
    if (xq_out && valid) *reinterpret_cast<uint4*>(xq_out + c0) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    if (xs_out && valid && (lane & 1) == 0) xs_out[c0 / QB] = s16;
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

// Routing as its own kernel (E > 64: a router workgroup holds only a 64-expert
// slice of its tokens' logits).  One workgroup per ROUTE_TILE tokens.  The
// routing fills few CUs, so the same launch also quantises the tokens: the
// n_tiles workgroups past the routing ones take ROUTE_TILE tokens each, one
// wavefront per token, writing the token-major codes and scales (and the
// shared-expert gate) that the bucketing launch would otherwise produce.
__global__ __launch_bounds__(ROUTE_WIDE_THREADS) void route_kernel(
    const float* __restrict__ logits, int n, int E, int k, int norm, int32_t* __restrict__ ids,
    float* __restrict__ wout, int32_t* __restrict__ rank, int32_t* __restrict__ hist, RowQuant rq) {
  const int n_tiles = (n + ROUTE_TILE - 1) / ROUTE_TILE;
  if ((int)blockIdx.x >= n_tiles) {
    const int lane = threadIdx.x & 63;
    const int t = ((int)blockIdx.x - n_tiles) * ROUTE_TILE + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (t < n)
      quantize_row(rq.x + (size_t)t * rq.d, rq.d, rq.d_pad, rq.shg, rq.gs + t, rq.xq + (size_t)t * rq.d_pad,
                   rq.xs + (size_t)t * (rq.d_pad / QB), rq.xq_out ? rq.xq_out + (size_t)t * rq.d : nullptr,
                   rq.xs_out ? rq.xs_out + (size_t)t * (rq.d / QB) : nullptr, lane);
    return;
  }
  __shared__ __attribute__((aligned(16))) RouteLds R;
  const int t0 = blockIdx.x * ROUTE_TILE;
  const int nt = min(ROUTE_TILE, n - t0);
  route_load_logits(R, logits, t0, nt, E, threadIdx.x);
  route_tile<MAX_EXPERTS / 64>(R, blockIdx.x, t0, nt, E, k, norm, threadIdx.x, ids, wout, rank, hist);
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
      quantize_row(x + (size_t)t * d, d, d_pad, shg, gs + t, xq + (size_t)t * d_pad,
                   xs + (size_t)t * (d_pad / QB), nullptr, nullptr, lane);
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


// The same logits for batches of 3..8 tokens, where decode_router_kernel's
// per-lane token reads bind (each lane reads its block's 16 quads for every
// token).  One workgroup per 16 experts, 8 wavefronts: in each pass of 2048 j
// row r of wavefront w (its 16 lanes are the 16 experts) chains block 4w + r
// for all NT tokens with its lanes' weight quads in registers, and the token
// values reach the row by DPP row broadcast inside the FMA (lane i of the row
// reads value i of each 16-j piece), so one LDS read serves 16 steps.  The
// block sums meet in LDS and thread (expert, token) adds them in block order.
constexpr int DRP_E = 16;  // experts per workgroup
template <int NT>
__global__ __launch_bounds__(512, 1) void decode_router_dpp_kernel(
    const float* __restrict__ x, int n, int d, int d_pad, const float* __restrict__ wt,
    const float* __restrict__ bias, int E, int E64, int n_rwg, float* __restrict__ logits,
    const float* __restrict__ shg, float* __restrict__ gs, int8_t* __restrict__ xq,
    uint16_t* __restrict__ xs) {
  __shared__ __attribute__((aligned(16))) float xl[NT][DR_JP];
  __shared__ __attribute__((aligned(16))) float part[NT][DRP_E][DR_NBP + 4];  // +4: bank offset per expert
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if ((int)blockIdx.x >= n_rwg) {
    const int t = (int)blockIdx.x - n_rwg;
    if (wave == 0 && t < n)
      quantize_row(x + (size_t)t * d, d, d_pad, shg, gs + t, xq + (size_t)t * d_pad,
                   xs + (size_t)t * (d_pad / QB), nullptr, nullptr, lane);
    return;
  }
  const int el = lane & 15, bl = 4 * wave + (lane >> 4);
  const int e = DRP_E * (int)blockIdx.x + el;  // < E64: the matrix holds zero rows past E
  const int se = tid % DRP_E, st = tid / DRP_E;
  float total = 0.0f;
  for (int j0 = 0; j0 < d; j0 += DR_JP) {
    // this pass's token values (thread tid: quad tid of every token; quads
    // past d skipped)
    f4v xv[NT];
    const bool xin = j0 + 4 * tid < d;
#pragma unroll
    for (int t = 0; t < NT; ++t)
      if (xin) xv[t] = *reinterpret_cast<const f4v*>(x + (size_t)t * d + j0 + 4 * tid);
    // this row's block: the lane's 16 weight quads (8 or none past d's last
    // full block; d % 32 == 0)
    const int jb = j0 + DR_RB * bl;
    const int nq = max(0, min(DR_RB, d - jb)) / 4;
    f4v w[DR_RB / 4];
#pragma unroll
    for (int q = 0; q < DR_RB / 4; ++q)
      if (q < nq) w[q] = *reinterpret_cast<const f4v*>(wt + ((size_t)(jb / 4 + q) * E64 + e) * 4);
    if (j0 > 0) __syncthreads();  // every lane is done with the previous pass's values and sums
#pragma unroll
    for (int t = 0; t < NT; ++t)
      if (xin) *reinterpret_cast<f4v*>(&xl[t][4 * tid]) = xv[t];
    __syncthreads();
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = 0.0f;
    const float* xb = &xl[0][DR_RB * bl] + el;
    auto piece = [&](int s) {  // 16 j: quads 4s .. 4s+3
#pragma unroll
      for (int t = 0; t + 1 < NT; t += 2)
        router_fma16_2(acc[t], acc[t + 1], xb[t * DR_JP + 16 * s], xb[(t + 1) * DR_JP + 16 * s], w[4 * s],
                       w[4 * s + 1], w[4 * s + 2], w[4 * s + 3]);
      if constexpr (NT % 2)
        router_fma16_1(acc[NT - 1], xb[(NT - 1) * DR_JP + 16 * s], w[4 * s], w[4 * s + 1], w[4 * s + 2],
                       w[4 * s + 3]);
    };
    if (nq > 0) {  // row-uniform; the DPP reads stay inside the row
      piece(0);
      piece(1);
      if (nq == DR_RB / 4) {
        piece(2);
        piece(3);
      }
    }
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
  const int eo = DRP_E * (int)blockIdx.x + se;
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
  dim3 grid((unsigned)((n + ROUTE_TILE - 1) / ROUTE_TILE), (unsigned)(E64 / 64));
  if ((long)grid.x * grid.y > n_cu)
    router_kernel<false, 1><<<grid, 512, 0, s>>>(x, n, d, wt, bias, E, E64, logits, 0, 0, nullptr, nullptr,
                                                 nullptr, nullptr);
  else
    router_kernel<false, 2><<<grid, 512, 0, s>>>(x, n, d, wt, bias, E, E64, logits, 0, 0, nullptr, nullptr,
                                                 nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_router_route(const float* x, int n, int d, const float* wt, const float* bias,
                               int E, int k, int norm, int32_t* ids, float* w, int32_t* rank,
                               int32_t* hist, int n_cu, hipStream_t s) {
  if (E > 64) return hipErrorInvalidValue;
  dim3 grid((unsigned)((n + ROUTE_TILE - 1) / ROUTE_TILE), 1);
  if ((long)grid.x > n_cu)
    router_kernel<true, 1><<<grid, 512, 0, s>>>(x, n, d, wt, bias, E, 64, nullptr, k, norm, ids, w, rank,
                                                hist);
  else
    router_kernel<true, 2><<<grid, 512, 0, s>>>(x, n, d, wt, bias, E, 64, nullptr, k, norm, ids, w, rank,
                                                hist);
  return hipGetLastError();
}

hipError_t launch_route(const float* logits, int n, int E, int k, int norm, int32_t* ids, float* w,
                        int32_t* rank, int32_t* hist, const RowQuant& rq, hipStream_t s) {
  const int tiles = (n + ROUTE_TILE - 1) / ROUTE_TILE;
  route_kernel<<<2 * tiles, ROUTE_WIDE_THREADS, 0, s>>>(logits, n, E, k, norm, ids, w, rank, hist, rq);
  return hipGetLastError();
}

hipError_t launch_decode_router(const float* x, int n, int d, int d_pad, const float* wt,
                                const float* bias, int E, int E64, float* logits,
                                const float* sh_gate_vec, float* gs, int8_t* dxq, uint16_t* dxs,
                                hipStream_t s) {
  if (n < 1 || n > DECODE_MAX_TOKENS) return hipErrorInvalidValue;
  // 1-2 tokens: lanes read their own token values (more workgroups stream the
  // matrix); 3-8: the DPP form (one LDS read per 16 steps)
  const int n_rwg = (E + DR_E - 1) / DR_E, n_rwg_dpp = (E + DRP_E - 1) / DRP_E;
#define DR_LAUNCH(NT)                                                                                  \
  case NT:                                                                                              \
    decode_router_kernel<NT><<<n_rwg + n, 256, 0, s>>>(x, n, d, d_pad, wt, bias, E, E64, n_rwg, logits,      \
                                                       sh_gate_vec, gs, dxq, dxs);                      \
    break;
#define DRP_LAUNCH(NT)                                                                                 \
  case NT:                                                                                              \
    decode_router_dpp_kernel<NT><<<n_rwg_dpp + n, 512, 0, s>>>(x, n, d, d_pad, wt, bias, E, E64, n_rwg_dpp,  \
                                                               logits, sh_gate_vec, gs, dxq, dxs);      \
    break;
  static_assert(DECODE_MAX_TOKENS == 8, "one instantiation per batch size");
  switch (n) {
    DR_LAUNCH(1) DR_LAUNCH(2) DRP_LAUNCH(3) DRP_LAUNCH(4) DRP_LAUNCH(5) DRP_LAUNCH(6) DRP_LAUNCH(7) DRP_LAUNCH(8)
  }
#undef DR_LAUNCH
#undef DRP_LAUNCH
  return hipGetLastError();
}

hipError_t launch_quantize(const float* v, int64_t n_values, int8_t* q, uint16_t* scales,
                           hipStream_t s) {
  const int64_t blocks = (n_values + 255) / 256;
  quantize_kernel<<<(unsigned)blocks, 256, 0, s>>>(v, n_values, q, scales);
  return hipGetLastError();
}

}  // namespace moe
