// bucket.hip -- expert bucketing on the GPU: the expStart / expTokI / expTokK
// CSR is built on the device, so the routing result never travels to the host
// between routing and the expert GEMMs (SharpInference #388, "Remaining
// levers" 1).
//
// The routing left, per 8-token tile, a histogram of expert counts and
// each (token, slot) pair's rank among the tile's pairs of the same expert.  A
// pair's CSR position is then
//     expStart[e] + (pairs of e in earlier tiles) + rank,
// which keeps every expert's rows in (token, slot) order -- a stable counting
// sort with no atomics, so the result is deterministic.  Each group's rows are
// cut into 128-row GEMM tiles, and each pair's token is also written at its
// tile row (first tile of its group * 128 + its index within the group), so
// that a GEMM workgroup finds its rows' tokens at an address given by its
// tile alone.  Workgroup 0 also writes expStart and the tile table that
// drives the grouped GEMMs.
//
// The same workgroup then quantises its tile's token rows (one launch for
// both stages: the rows' loads are issued before the histograms are read, so
// their latency hides under the bucketing).  One wavefront per token: lane
// pairs quantise 32-blocks (each lane 16 values).  Each block's codes are
// written once, token-major (gq[token][d_pad]), and the gate/up GEMM gathers
// its tiles' rows from there; each block's scale is written once per expert
// slot of the token, in the GEMM's scale layout at the slot's tile row
// (t32 = row / 32, r = row % 32): gqs[t32][k-step][r][block].  The K-padding
// blocks past d get zero codes and scales.  With a shared expert
// the wavefront also computes the gate sigmoid(x . g) (a fixed-order
// reduction).  Optionally the token-major codes and scales of the unpadded
// width d are written out as well.
#include "device_util.h"
#include "internal.h"

namespace moe {
namespace {

// Exclusive prefix sum of up to 512 ints held in s[0..n), in place, by one
// wavefront (call from all 64 lanes of one wavefront): 8 values per lane, then a
// shuffle scan of the 64 lane totals.
__device__ void wave_exclusive_scan_512(int* s, int n, int lane) {
  int v[8];
  int tot = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int i = lane * 8 + j;
    v[j] = (i < n) ? s[i] : 0;
    tot += v[j];
  }
  int inc = tot;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int up = __shfl_up(inc, off, 64);
    if (lane >= off) inc += up;
  }
  int run = inc - tot;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int i = lane * 8 + j;
    if (i < n) s[i] = run;
    run += v[j];
  }
}

typedef float f4v __attribute__((ext_vector_type(4)));
constexpr int BQ_THREADS = 64 * ROUTE_TILE;  // a wavefront per token of the tile

struct QuantArgs {
  const float* x;
  int d, d_pad;
  int8_t* gq;
  uint16_t* gqs;
  const float* shg;  // shared-expert gate vector, or NULL
  float* gs;
  int8_t* xq_out;    // optional token-major copies
  uint16_t* xs_out;
  const uint16_t* xs_tok;  // non-NULL: the codes are written, these are their scales
};

// At most 128 VGPRs (four wavefronts per SIMD), so that two 512-thread
// workgroups share a CU when there are more tiles than CUs.
__global__ __launch_bounds__(BQ_THREADS) __attribute__((amdgpu_waves_per_eu(4, 8))) void bucket_quantize_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ rank,
    const int32_t* __restrict__ hist, int n, int E, int k, int has_shared, int n_tiles,
    int32_t* __restrict__ exp_start, int32_t* __restrict__ tok_i, int32_t* __restrict__ tok_k,
    int32_t* __restrict__ row_tok, int32_t* __restrict__ tiles, int tile_bound, QuantArgs qa) {
  __shared__ int s_start[2 * 256 + 2];
  __shared__ int s_pre[MAX_EXPERTS];
  __shared__ int s_cnt[MAX_EXPERTS + 1];
  __shared__ int s_nt[2 * 256 + 2];
  __shared__ int s_pos[ROUTE_TILE][MAX_TOPK + 1];
  const int tile = blockIdx.x;
  const int P = n * k;
  const int G = E + has_shared;
  const int kk = k + has_shared;
  const int t0 = tile * ROUTE_TILE;
  const int nt = min(ROUTE_TILE, n - t0);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // This wavefront's token row (the last one for a wavefront past the tile's
  // tokens, which quantises nothing): the values of its first two passes of
  // 8 k-steps are requested now (padding columns load column 0 and are
  // zeroed later).
  const int tq = t0 + min(wave, nt - 1);
  const float* xr = qa.x + (size_t)tq * qa.d;
  const int KS = qa.d_pad / (QB * KSTEP);
  auto load = [&](int j0, f4v (&v)[4]) {
    const int j = j0 + (lane >> 3), p = lane & 7;
    const int c0 = (KSTEP * j + (p >> 1)) * QB + (p & 1) * 16;
    const float* src = xr + (c0 < qa.d ? c0 : 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = *reinterpret_cast<const f4v*>(src + 4 * i);
  };
  f4v cur[4] = {}, nxt[4] = {};
  if (!qa.xs_tok) {
    load(0, cur);
    if (8 < KS) load(8, nxt);
  }

  // Per-expert totals over all tiles and over the tiles before this one; for
  // small E several threads share an expert's column and their sums meet in LDS.
  __shared__ int s_part_tot[BQ_THREADS], s_part_pre[BQ_THREADS];
  const int nparts = max(1, BQ_THREADS / E);
  // Every workgroup reads every histogram, so this is the kernel's critical
  // path: a thread requests RB histogram entries at once (the index clamped
  // into the table, the surplus masked), one memory round trip per RB tiles.
  constexpr int RB = 32;
  if (threadIdx.x < E * nparts) {
    const int e = threadIdx.x % E, part = threadIdx.x / E;
    int tot = 0, pre = 0;
    for (int tt = part; tt < n_tiles; tt += RB * nparts) {
      int h[RB];
#pragma unroll
      for (int u = 0; u < RB; ++u) h[u] = hist[(size_t)min(tt + u * nparts, n_tiles - 1) * E + e];
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        const int tu = tt + u * nparts;
        tot += (tu < n_tiles) ? h[u] : 0;
        pre += (tu < tile) ? h[u] : 0;
      }
    }
    s_part_tot[threadIdx.x] = tot;
    s_part_pre[threadIdx.x] = pre;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += BQ_THREADS) {
    int tot = 0, pre = 0;
    for (int part = 0; part < nparts; ++part) {
      tot += s_part_tot[part * E + e];
      pre += s_part_pre[part * E + e];
    }
    s_start[e] = tot;
    s_cnt[e] = tot;
    s_pre[e] = pre;
  }
  if (threadIdx.x == 0 && has_shared) s_cnt[E] = n;
  __syncthreads();
  // group tile counts (every workgroup needs the first tile of each group)
  for (int g = threadIdx.x; g < G; g += BQ_THREADS) s_nt[g] = (s_cnt[g] + MT_WG - 1) / MT_WG;
  __syncthreads();
  const int last_nt = s_nt[G - 1];
  __syncthreads();
  if (threadIdx.x < 64) wave_exclusive_scan_512(s_start, E, threadIdx.x);
  else if (threadIdx.x < 128) wave_exclusive_scan_512(s_nt, G, threadIdx.x - 64);
  __syncthreads();

  // Each pair's CSR row, and its token at its tile row: row i of tile T
  // (T * 128 + i) is CSR row (first row of T) + i, so a pair at index `local`
  // within group e sits at tile row (first tile of e) * 128 + local.
  const int pad_rows = tile_bound * MT_WG;
  for (int q = threadIdx.x; q < nt * k; q += BQ_THREADS) {
    const int t = t0 + q / k, s = q % k;
    const int e = ids[(size_t)t * k + s];
    const int local = s_pre[e] + rank[(size_t)t * k + s];
    const int pos = s_start[e] + local;
    if ((unsigned)pos < (unsigned)P) {
      tok_i[pos] = t;
      tok_k[pos] = s;
    }
    const int prow = s_nt[e] * MT_WG + local;
    if (prow < pad_rows) row_tok[prow] = t;
    s_pos[q / k][s] = prow < pad_rows ? prow : -1;
  }
  if (has_shared)
    for (int q = threadIdx.x; q < nt; q += BQ_THREADS) {
      tok_i[P + t0 + q] = t0 + q;
      tok_k[P + t0 + q] = k;
      const int prow = s_nt[E] * MT_WG + t0 + q;
      if (prow < pad_rows) row_tok[prow] = t0 + q;
      s_pos[q][k] = prow < pad_rows ? prow : -1;
    }

  if (tile == 0) {
    // expStart, then the 128-row tile table over the E (+1) groups
    for (int e = threadIdx.x; e <= E; e += BQ_THREADS) exp_start[e] = (e < E) ? s_start[e] : P;
    if (has_shared && threadIdx.x == 0) exp_start[E + 1] = P + n;
    for (int g = threadIdx.x; g < G; g += BQ_THREADS) {
      const int c = s_cnt[g];
      const int first = (g < E) ? s_start[g] : P;
      const int ntg = (c + MT_WG - 1) / MT_WG;
      for (int i = 0; i < ntg && s_nt[g] + i < tile_bound; ++i) {
        int32_t* ent = tiles + 4 + 3 * (size_t)(s_nt[g] + i);
        ent[0] = g;
        ent[1] = first + i * MT_WG;
        ent[2] = first + c;
      }
    }
    if (threadIdx.x == 0) {
      tiles[0] = min(s_nt[G - 1] + last_nt, tile_bound);
      tiles[1] = 0;
      tiles[2] = 0;
      tiles[3] = 0;
    }
  }
  __syncthreads();  // the tile's padded rows are in s_pos

  // Quantise: wavefront w takes token t0 + w.
  if (wave >= nt) return;
  const int t = t0 + wave;
  // The k-step's 4 scales, once per expert slot at the slot's tile row: lane
  // p of the k-step's 8 takes slots p and p + 8.
  auto place_scales = [&](int j, int p, uint2 sc4) {
    for (int s2 = p; s2 < kk; s2 += 8) {
      const int row = s_pos[wave][s2];
      if (row >= 0)
        *reinterpret_cast<uint2*>(qa.gqs + (((size_t)(row >> 5) * KS + j) * 32 + (row & 31)) * KSTEP) = sc4;
    }
  };
  if (qa.xs_tok) {
    for (int j0 = 0; j0 < KS; j0 += 8) {
      const int j = j0 + (lane >> 3);
      if (j < KS)
        place_scales(j, lane & 7,
                     *reinterpret_cast<const uint2*>(qa.xs_tok + (size_t)t * (qa.d_pad / QB) + KSTEP * j));
    }
    return;
  }
  float gacc = 0.0f;
  // Each pass covers 8 k-steps; the pass after next is requested before this
  // pass is quantised and stored.
  for (int j0 = 0; j0 < KS; j0 += 8) {
    f4v nn[4] = {};
    if (j0 + 16 < KS) load(j0 + 16, nn);
    const int j = j0 + (lane >> 3), p = lane & 7;  // k-step, piece
    const int kb = KSTEP * j + (p >> 1), half = p & 1;
    const int c0 = kb * QB + half * 16;  // first column of the piece
    const bool valid = c0 < qa.d;        // d % 32 == 0: a piece is all valid or all padding
    float v[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[4 * i] = valid ? cur[i].x : 0.0f;
      v[4 * i + 1] = valid ? cur[i].y : 0.0f;
      v[4 * i + 2] = valid ? cur[i].z : 0.0f;
      v[4 * i + 3] = valid ? cur[i].w : 0.0f;
    }
    uint32_t pk[4];
    uint16_t s16;
    quant_half_block16(v, pk, s16);  // lanes 2i, 2i+1 share a block; all take part
    // the k-step's 4 scales (held by lanes 0, 2, 4, 6 of its 8) in every lane
    const int g8 = lane & ~7;
    const uint32_t sb0 = (uint32_t)__shfl((int)s16, g8, 64), sb1 = (uint32_t)__shfl((int)s16, g8 + 2, 64);
    const uint32_t sb2 = (uint32_t)__shfl((int)s16, g8 + 4, 64), sb3 = (uint32_t)__shfl((int)s16, g8 + 6, 64);
    if (j < KS) {
      const uint4 codes = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      *reinterpret_cast<uint4*>(qa.gq + (size_t)t * qa.d_pad + c0) = codes;
      place_scales(j, p, make_uint2(sb0 | (sb1 << 16), sb2 | (sb3 << 16)));
      if (qa.xq_out && valid) *reinterpret_cast<uint4*>(qa.xq_out + (size_t)t * qa.d + c0) = codes;
      if (qa.xs_out && half == 0 && valid) qa.xs_out[(size_t)t * (qa.d / QB) + kb] = s16;
    }
    if (qa.shg && valid) {
#pragma unroll
      for (int i = 0; i < 16; ++i) gacc = __builtin_fmaf(v[i], qa.shg[c0 + i], gacc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      cur[i] = nxt[i];
      nxt[i] = nn[i];
    }
  }
  if (qa.shg) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) gacc += __shfl_xor(gacc, off, 64);
    if (lane == 0) qa.gs[t] = 1.0f / (1.0f + expf(-gacc));
  }
}

}  // namespace

hipError_t launch_bucket_quantize(const int32_t* ids, const int32_t* rank, const int32_t* hist, int n,
                                  int E, int k, int has_shared, int32_t* exp_start, int32_t* tok_i,
                                  int32_t* tok_k, int32_t* row_tok, int32_t* tiles, int tile_bound,
                                  const float* x, int d, int d_pad, int8_t* gq, uint16_t* gqs,
                                  const float* sh_gate_vec, float* gs, int8_t* xq_out, uint16_t* xs_out,
                                  const uint16_t* xs_tok, hipStream_t s) {
  const int n_tiles = (n + ROUTE_TILE - 1) / ROUTE_TILE;
  const QuantArgs qa{x, d, d_pad, gq, gqs, sh_gate_vec, gs, xq_out, xs_out, xs_tok};
  bucket_quantize_kernel<<<n_tiles, BQ_THREADS, 0, s>>>(ids, rank, hist, n, E, k, has_shared, n_tiles, exp_start,
                                                        tok_i, tok_k, row_tok, tiles, tile_bound, qa);
  return hipGetLastError();
}

}  // namespace moe
