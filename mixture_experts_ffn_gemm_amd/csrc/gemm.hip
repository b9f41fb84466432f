// gemm.hip -- the two grouped int8 expert GEMMs, each a single launch over
// every expert group (routed experts and, as group E, the shared expert).
//
// SharpInference #406 "The work" item 2 asks for a grouped/segmented expert GEMM
// (gather tokens per expert -> GEMM -> scatter) instead of per-token matvecs, and
// #388 "Remaining levers" 3 replaces 256 per-expert GEMM launches per layer with
// one grouped GEMM over all experts.  The int8 MMQ contract of #406 ("Q8_0 MMQ",
// argmax-stable) fixes the arithmetic: exact int32 sums per 32-block, scaled by
// activation-scale * weight-scale and accumulated in fp32.
//
// Work decomposition: the bucketing kernel writes a table of 32-row tiles (a
// tile never straddles two groups).  A work item is one wavefront computing one
// tile against one column strip; items are numbered column-strip-major so that
// consecutive items -- the same workgroup, the same XCD -- share the weight strip
// through L2.  The grid is the static upper bound on the number of items;
// surplus wavefronts exit after reading the tile count.
//
// Per 32-block k-step a wavefront issues one v_mfma_i32_32x32x32_i8 per 32x32
// output tile (A: lane l holds row l%32, bytes 16*(l/32)..+15 of the block; B:
// the same for the weight row; D: lane l holds column l%32 of rows
// 8*(v/4) + 4*(l/32) + v%4 in register v), then rescales the int32 result into
// the fp32 accumulator with the product of the two binary16 block scales.
#include "device_util.h"
#include "internal.h"

namespace moe {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

__device__ inline int out_row(int v, int lane) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }

__device__ inline float h2f(uint16_t b) { return __half2float(__ushort_as_half(b)); }

// acc[tt] += scale-corrected int32 block products, tt = 0..3 tiles sharing the A rows.
__device__ inline void mfma_rescale4(const v4i& av, const v4i (&bv)[4], const float (&sa)[16],
                                     const float (&sw)[4], v16f (&acc)[4]) {
  const v16i zero = {0};
  v16i c[4];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) c[tt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, bv[tt], zero, 0, 0, 0);
#pragma unroll
  for (int tt = 0; tt < 4; ++tt)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[tt][v] = __builtin_fmaf((float)c[tt][v], sa[v] * sw[tt], acc[tt][v]);
}

// Loads the four 16-byte-per-lane activation scales of a k-step (4 blocks) for
// this lane's A row and spreads them to the 16 output rows this lane holds.
__device__ inline void spread_row_scales(uint2 packed, int lane, float (&sa)[4][16]) {
  const float s0 = h2f((uint16_t)(packed.x & 0xffffu));
  const float s1 = h2f((uint16_t)(packed.x >> 16));
  const float s2 = h2f((uint16_t)(packed.y & 0xffffu));
  const float s3 = h2f((uint16_t)(packed.y >> 16));
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int src = out_row(v, lane);
    sa[0][v] = __shfl(s0, src, 64);
    sa[1][v] = __shfl(s1, src, 64);
    sa[2][v] = __shfl(s2, src, 64);
    sa[3][v] = __shfl(s3, src, 64);
  }
}

__device__ inline void unpack_scales(uint2 packed, float (&s)[4]) {
  s[0] = h2f((uint16_t)(packed.x & 0xffffu));
  s[1] = h2f((uint16_t)(packed.x >> 16));
  s[2] = h2f((uint16_t)(packed.y & 0xffffu));
  s[3] = h2f((uint16_t)(packed.y >> 16));
}

// Gate/up + SwiGLU + per-32 requantisation.  Item = (64 SwiGLU columns, one
// 32-row tile).  Tiles 0,1 of the strip are gate rows, 2,3 the matching up rows,
// so h = silu(gate) * up is formed lane by lane.  The int8 h codes are written
// as the down GEMM's A-operand chunks of the same tile.
__global__ __launch_bounds__(256, 2) void gateup_kernel(GemmArgs a) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int item = xcd_major(blockIdx.x, gridDim.x) * 4 + wv;
  const int n_tiles = min(a.tiles[0], a.tile_bound);
  const int nct_max = max(a.F_pad, a.Fs_pad) / GU_COLS;
  if (item >= n_tiles * nct_max) return;
  const int c = item / n_tiles, T = item - (item / n_tiles) * n_tiles;
  const int32_t* ent = a.tiles + 4 + 3 * T;
  const int g = ent[0], row0 = ent[1], row_end = ent[2];
  if (g < 0 || g >= a.G || row0 < 0 || row_end <= row0 || row_end > a.p_total) return;
  const bool shared = g >= a.E;
  const int Fg_pad = shared ? a.Fs_pad : a.F_pad;
  if (c >= Fg_pad / GU_COLS) return;
  const int KB = a.d_pad / QB;

  const int8_t* bq = (shared ? a.sh_gu_q : a.gu_q + (size_t)g * a.gu_q_group) +
                     (size_t)c * KB * 4096 + lane * 16;
  const uint16_t* bs = (shared ? a.sh_gu_s : a.gu_s + (size_t)g * a.gu_s_group) +
                       ((size_t)c * 4 * 32 + (lane & 31)) * KB;
  const int p_lane = min(row0 + (lane & 31), row_end - 1);
  const int tok = min(max(a.tok_i[p_lane], 0), a.n_tokens - 1);
  const int8_t* ap = a.xq + (size_t)tok * a.d_pad + (lane >> 5) * 16;
  const uint16_t* asp = a.xs + (size_t)tok * KB;

  v16f acc[4];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) acc[tt] = (v16f){0};

  for (int kb0 = 0; kb0 < KB; kb0 += 4) {
    float sa[4][16];
    spread_row_scales(*reinterpret_cast<const uint2*>(asp + kb0), lane, sa);
    float swt[4][4];  // [tile][block]
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
      unpack_scales(*reinterpret_cast<const uint2*>(bs + (size_t)tt * 32 * KB + kb0), swt[tt]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kb = kb0 + i;
      const v4i av = *reinterpret_cast<const v4i*>(ap + kb * QB);
      v4i bv[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) bv[tt] = *reinterpret_cast<const v4i*>(bq + (size_t)(kb * 4 + tt) * 1024);
      const float sw[4] = {swt[0][i], swt[1][i], swt[2][i], swt[3][i]};
      mfma_rescale4(av, bv, sa[i], sw, acc);
    }
  }

  // SwiGLU and requantisation, one 32-column block per sub-strip.
  int8_t* hq_tile = a.hq + (size_t)T * a.kbmax * 1024;
  uint16_t* hs_tile = a.hs + (size_t)T * 32 * a.kbmax;
  const int cb = lane & 31;
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    const int kbf = 2 * c + sub;
    int8_t* chunk = hq_tile + (size_t)kbf * 1024 + (cb >> 4) * 512 + (cb & 15);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float gv = acc[sub][v], uv = acc[2 + sub][v];
      const float h = gv / (1.0f + expf(-gv)) * uv;
      int8_t q;
      uint16_t s16;
      quant_block32(h, q, s16);
      const int m = out_row(v, lane);
      chunk[m * 16] = q;
      if (cb == 0) hs_tile[(size_t)m * a.kbmax + kbf] = s16;
    }
  }
}

// Down projection.  Item = (128 output columns, one 32-row tile); the fp32
// result rows are the unweighted down-partials (#129 "Scope"), scattered to
// partial[token][slot] through expTokI / expTokK.
__global__ __launch_bounds__(256, 2) void down_kernel(GemmArgs a) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int item = xcd_major(blockIdx.x, gridDim.x) * 4 + wv;
  const int n_tiles = min(a.tiles[0], a.tile_bound);
  const int nct = a.d_pad / DN_COLS;
  if (item >= n_tiles * nct) return;
  const int c = item / n_tiles, T = item - (item / n_tiles) * n_tiles;
  const int32_t* ent = a.tiles + 4 + 3 * T;
  const int g = ent[0], row0 = ent[1], row_end = ent[2];
  if (g < 0 || g >= a.G || row0 < 0 || row_end <= row0 || row_end > a.p_total) return;
  const bool shared = g >= a.E;
  const int KB = (shared ? a.Fs_pad : a.F_pad) / QB;

  const int8_t* bq = (shared ? a.sh_dn_q : a.dn_q + (size_t)g * a.dn_q_group) +
                     (size_t)c * KB * 4096 + lane * 16;
  const uint16_t* bs = (shared ? a.sh_dn_s : a.dn_s + (size_t)g * a.dn_s_group) +
                       ((size_t)c * 4 * 32 + (lane & 31)) * KB;
  const int8_t* ap = a.hq + (size_t)T * a.kbmax * 1024 + lane * 16;
  const uint16_t* asp = a.hs + ((size_t)T * 32 + (lane & 31)) * a.kbmax;

  v16f acc[4];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) acc[tt] = (v16f){0};

  for (int kb0 = 0; kb0 < KB; kb0 += 4) {
    float sa[4][16];
    spread_row_scales(*reinterpret_cast<const uint2*>(asp + kb0), lane, sa);
    float swt[4][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
      unpack_scales(*reinterpret_cast<const uint2*>(bs + (size_t)tt * 32 * KB + kb0), swt[tt]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kb = kb0 + i;
      const v4i av = *reinterpret_cast<const v4i*>(ap + (size_t)kb * 1024);
      v4i bv[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) bv[tt] = *reinterpret_cast<const v4i*>(bq + (size_t)(kb * 4 + tt) * 1024);
      const float sw[4] = {swt[0][i], swt[1][i], swt[2][i], swt[3][i]};
      mfma_rescale4(av, bv, sa[i], sw, acc);
    }
  }

  const int p_lane = min(row0 + (lane & 31), row_end - 1);
  const int tok_l = a.tok_i[p_lane];
  const int slot_l = a.tok_k[p_lane];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int m = out_row(v, lane);
    const int tok = __shfl(tok_l, m, 64);
    const int slot = __shfl(slot_l, m, 64);
    if (row0 + m < row_end && (unsigned)tok < (unsigned)a.n_tokens && (unsigned)slot < (unsigned)a.kk) {
      float* dst = a.partial + ((size_t)tok * a.kk + slot) * a.d;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int col = c * DN_COLS + tt * 32 + (lane & 31);
        if (col < a.d) dst[col] = acc[tt][v];
      }
    }
  }
}

int grid_for_items(long items) {
  long wgs = (items + 3) / 4;
  wgs = (wgs + 7) / 8 * 8;
  return (int)wgs;
}

}  // namespace

hipError_t launch_gateup(const GemmArgs& a, hipStream_t s) {
  const long items = (long)a.tile_bound * (max(a.F_pad, a.Fs_pad) / GU_COLS);
  gateup_kernel<<<grid_for_items(items), 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_down(const GemmArgs& a, hipStream_t s) {
  const long items = (long)a.tile_bound * (a.d_pad / DN_COLS);
  down_kernel<<<grid_for_items(items), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
