// bucket.hip -- expert bucketing on the GPU (SharpInference #388 "Remaining
// levers" 1: the expStart / expTokI / expTokK CSR must be built on the GPU or the
// selection round-trips to the host).
//
// The routing kernel left, per 16-token tile, a histogram of expert counts and
// each (token, slot) pair's rank among the tile's pairs of the same expert.  A
// pair's CSR position is then
//     expStart[e] + (pairs of e in earlier tiles) + rank,
// which keeps every expert's rows in (token, slot) order -- a stable counting
// sort with no atomics, so the result is deterministic.  Each group's rows are
// cut into 128-row GEMM tiles; a pair's padded row (its group's first tile *
// 128 + its index within the group) is written per (token, slot), so the
// quantiser can place the token's codes where the GEMM's tile reads them.
// Workgroup 0 also writes expStart and the tile table that drives the grouped
// GEMMs.
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

__global__ __launch_bounds__(256) void bucket_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ rank,
    const int32_t* __restrict__ hist, int n, int E, int k, int has_shared, int n_tiles,
    int32_t* __restrict__ exp_start, int32_t* __restrict__ tok_i, int32_t* __restrict__ tok_k,
    int32_t* __restrict__ pos_out, int32_t* __restrict__ tiles, int tile_bound) {
  __shared__ int s_start[2 * 256 + 2];
  __shared__ int s_pre[MAX_EXPERTS];
  __shared__ int s_cnt[MAX_EXPERTS + 1];
  __shared__ int s_nt[2 * 256 + 2];
  const int tile = blockIdx.x;
  const int P = n * k;
  const int G = E + has_shared;
  const int kk = k + has_shared;
  // Per-expert totals over all tiles and over the tiles before this one; for
  // small E several threads share an expert's column and their sums meet in LDS.
  __shared__ int s_part_tot[256], s_part_pre[256];
  const int nparts = max(1, 256 / E);
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
  for (int e = threadIdx.x; e < E; e += 256) {
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
  for (int g = threadIdx.x; g < G; g += 256) s_nt[g] = (s_cnt[g] + MT_WG - 1) / MT_WG;
  __syncthreads();
  const int last_nt = s_nt[G - 1];
  __syncthreads();
  if (threadIdx.x < 64) wave_exclusive_scan_512(s_start, E, threadIdx.x);
  else if (threadIdx.x < 128) wave_exclusive_scan_512(s_nt, G, threadIdx.x - 64);
  __syncthreads();

  const int pad_rows = tile_bound * MT_WG;
  const int t0 = tile * ROUTE_TILE;
  const int nt = min(ROUTE_TILE, n - t0);
  for (int q = threadIdx.x; q < nt * k; q += 256) {
    const int t = t0 + q / k, s = q % k;
    const int e = ids[(size_t)t * k + s];
    const int local = s_pre[e] + rank[(size_t)t * k + s];
    const int pos = s_start[e] + local;
    if ((unsigned)pos < (unsigned)P) {
      tok_i[pos] = t;
      tok_k[pos] = s;
    }
    const int prow = s_nt[e] * MT_WG + local;
    pos_out[(size_t)t * kk + s] = prow < pad_rows ? prow : -1;
  }
  if (has_shared)
    for (int q = threadIdx.x; q < nt; q += 256) {
      tok_i[P + t0 + q] = t0 + q;
      tok_k[P + t0 + q] = k;
      const int prow = s_nt[E] * MT_WG + t0 + q;
      pos_out[(size_t)(t0 + q) * kk + k] = prow < pad_rows ? prow : -1;
    }

  if (tile != 0) return;
  // expStart, then the 128-row tile table over the E (+1) groups
  for (int e = threadIdx.x; e <= E; e += 256) exp_start[e] = (e < E) ? s_start[e] : P;
  if (has_shared && threadIdx.x == 0) exp_start[E + 1] = P + n;
  for (int g = threadIdx.x; g < G; g += 256) {
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

}  // namespace

hipError_t launch_bucket(const int32_t* ids, const int32_t* rank, const int32_t* hist, int n, int E,
                         int k, int has_shared, int32_t* exp_start, int32_t* tok_i, int32_t* tok_k,
                         int32_t* pos, int32_t* tiles, int tile_bound, hipStream_t s) {
  const int n_tiles = (n + ROUTE_TILE - 1) / ROUTE_TILE;
  bucket_kernel<<<n_tiles, 256, 0, s>>>(ids, rank, hist, n, E, k, has_shared, n_tiles, exp_start,
                                        tok_i, tok_k, pos, tiles, tile_bound);
  return hipGetLastError();
}

}  // namespace moe
