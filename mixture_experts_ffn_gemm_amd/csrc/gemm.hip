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
// Work decomposition: the bucketing kernel writes a table of 128-row tiles (a
// tile never straddles two groups).  A workgroup (4 wavefronts, 32 rows each)
// computes one tile against one column strip.  Workgroups are numbered
// tile-major (strips inner) and dealt to the 8 XCDs in contiguous ranges, so
// one XCD runs every strip of a tile back to back (the tile's activation rows
// stay in its L2) and the few tiles of one expert mostly share an XCD (each
// weight strip is fetched about once).  The grid is the static upper bound on
// the number of workgroups; surplus workgroups exit after reading the tile
// count.
//
// K loop: per k-step of 4 blocks the workgroup stages the strip's weight codes
// (4 blocks x 4 tiles of 32x32 bytes) and their binary16 scales (17 KiB) in LDS
// with direct global->LDS loads, double-buffered.  Per 32-block each wavefront
// issues, per 32x32 output tile,
//   v_mfma_i32_32x32x32_i8  -> exact int32 block sums C[m][n]
//   v_mfma_f32_32x32x8_f16  -> S[m][n] = sa[m] * sw[n]: an outer product of the
//                              two binary16 block scales, exact in fp32 (only
//                              one of the 8 K slots is non-zero in A),
// and the VALU does acc = fma(float(C), S, acc): two VALU operations per
// output element per block, which is the bound of this kernel (the MFMA pipe
// is about 35% busy).
// Operand layouts (gfx950): A lane l = row l%32, bytes/halves k = 16*(l/32)+j
// (i8) or 4*(l/32)+j (f16x8); B likewise by column; D lane l = column l%32,
// register v = row 8*(v/4) + 4*(l/32) + v%4.
#include "device_util.h"
#include "internal.h"

namespace moe {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

constexpr int A_OFF = KSTEP_BYTES;                   // A chunks follow the weight k-step
constexpr int STAGE_BYTES = KSTEP_BYTES + 4 * KSTEP * 1024;  // + 4 wavefronts x 4 A chunks

__device__ inline int out_row(int v, int lane) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }

__device__ inline v4h as_v4h(uint32_t lo, uint32_t hi) {
  const uint2 u = make_uint2(lo, hi);
  return __builtin_bit_cast(v4h, u);
}

// Stage k-step `ks`: the weight strip's 17 chunks of 1 KiB (codes + scales)
// into `dst`, and this wavefront's 4 A-operand chunks (one per block) into
// dst + A_OFF + wave * 4 KiB.  All loads go straight from global memory to LDS;
// A rows are gathered per lane (lane l supplies row l%32, half l/32).
__device__ inline void stage_kstep(const uint8_t* strip, int ks, const int8_t* ap, size_t a_blk,
                                   char* dst, int wave, int lane) {
  const uint8_t* src = strip + (size_t)ks * KSTEP_BYTES + lane * 16;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int chunk = wave + 4 * i;
    __builtin_amdgcn_global_load_lds((glb_void*)(src + chunk * 1024), (lds_void*)(dst + chunk * 1024), 16, 0, 0);
  }
  if (wave == 0)
    __builtin_amdgcn_global_load_lds((glb_void*)(src + 16 * 1024), (lds_void*)(dst + 16 * 1024), 16, 0, 0);
  const int8_t* as = ap + (size_t)ks * KSTEP * a_blk;
  char* ad = dst + A_OFF + wave * (KSTEP * 1024);
#pragma unroll
  for (int i = 0; i < KSTEP; ++i)
    __builtin_amdgcn_global_load_lds((glb_void*)(as + i * a_blk), (lds_void*)(ad + i * 1024), 16, 0, 0);
}

// Operands of one k-step (4 blocks x 4 output tiles) for this wavefront, read
// from the staged LDS buffer into registers: the A chunks of its 32 rows, the
// 16 B chunks and the weight scales of the 4 tiles.
struct KOps {
  v4i av[KSTEP];
  v4i bv[4 * KSTEP];
  v4h sw[4];
};

__device__ inline void load_kstep(const char* buf, int wave, int lane, KOps& o) {
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const uint2 p = *reinterpret_cast<const uint2*>(buf + 16 * 1024 + (tt * 32 + (lane & 31)) * 8);
    o.sw[tt] = as_v4h(p.x, p.y);
  }
  const char* bp = buf + lane * 16;
  const char* apl = buf + A_OFF + wave * (KSTEP * 1024) + lane * 16;
#pragma unroll
  for (int i = 0; i < KSTEP; ++i) o.av[i] = *reinterpret_cast<const v4i*>(apl + i * 1024);
#pragma unroll
  for (int j = 0; j < 4 * KSTEP; ++j) o.bv[j] = *reinterpret_cast<const v4i*>(bp + j * 1024);
}

// One k-step from registers.  sa holds the 4 binary16 activation scales of
// this lane's A row; lanes 32..63 contribute zero K slots to the scale MFMA.
// The 16 (block, tile) steps are software-pipelined one step deep with the
// issue order pinned so that every MFMA is followed by 16 independent VALU
// operations of the previous step: the MFMA pipe (about half as busy as the
// VALU) then never blocks instruction issue.
__device__ inline void compute_kstep(const KOps& o, uint2 sa, int lane, v16f (&acc)[4]) {
  const v16i zi = {0};
  const v16f zf = {0};
  if (lane >= 32) sa = make_uint2(0u, 0u);
  v4h sav[KSTEP];
#pragma unroll
  for (int i = 0; i < KSTEP; ++i) {
    const uint32_t m = (i & 1) ? 0xffff0000u : 0x0000ffffu;
    sav[i] = (i < 2) ? as_v4h(sa.x & m, 0u) : as_v4h(0u, sa.y & m);
  }
  v16i c_cur = __builtin_amdgcn_mfma_i32_32x32x32_i8(o.av[0], o.bv[0], zi, 0, 0, 0);
  v16f s_cur = __builtin_amdgcn_mfma_f32_32x32x8f16(sav[0], o.sw[0], zf, 0, 0, 0);
#pragma unroll
  for (int j = 0; j < 4 * KSTEP; ++j) {
    const int t0 = j & 3;
    const bool more = j + 1 < 4 * KSTEP;
    const int i1 = (j + 1) >> 2, t1 = (j + 1) & 3;
    v16i c_nxt;
    v16f s_nxt;
    float cf[16];
    // sched_barrier(0) fences pin this exact order: MFMA(j+1), convert(j),
    // scale MFMA(j+1), accumulate(j).
    if (more) c_nxt = __builtin_amdgcn_mfma_i32_32x32x32_i8(o.av[i1], o.bv[j + 1], zi, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int v = 0; v < 16; ++v) cf[v] = (float)c_cur[v];
    __builtin_amdgcn_sched_barrier(0);
    if (more) s_nxt = __builtin_amdgcn_mfma_f32_32x32x8f16(sav[i1], o.sw[t1], zf, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[t0][v] = __builtin_fmaf(cf[v], s_cur[v], acc[t0][v]);
    __builtin_amdgcn_sched_barrier(0);
    if (more) {
      c_cur = c_nxt;
      s_cur = s_nxt;
    }
  }
}

// One iteration of the double-buffered k loop on buffer `cur` (the other
// buffer, `nxt`, receives k-step ks+1).  Order matters: the barrier makes
// k-step ks visible and frees `nxt` (every wavefront has read its operands of
// ks-1); the operands of ks are read into registers before the loads into
// `nxt` are issued, so no LDS read waits behind those loads; the prefetched
// activation scales are first used one iteration later, so nothing waits for
// them either.  The loads of ks+1 then overlap the whole compute of ks.
__device__ inline void kloop_step(const uint8_t* strip, int ks, int KS, const int8_t* ap, size_t a_blk,
                                  const uint16_t* asp, bool active, int wave, int lane,
                                  const char* cur, char* nxt, uint2 sa_cur, uint2& sa_nxt,
                                  v16f (&acc)[4]) {
  __syncthreads();
  KOps o;
  if (active) load_kstep(cur, wave, lane, o);
  if (ks + 1 < KS) {
    stage_kstep(strip, ks + 1, ap, a_blk, nxt, wave, lane);
    if (active) sa_nxt = *reinterpret_cast<const uint2*>(asp + (size_t)(ks + 1) * KSTEP);
  }
  if (active) compute_kstep(o, sa_cur, lane, acc);
}

// Grouped GEMM.  GATEUP: A = gathered int8 token rows (xq via expTokI), B = the
// [gate;up] strip of 64 SwiGLU columns; epilogue h = silu(gate) * up,
// requantised per 32 into the down GEMM's A-operand chunks.  !GATEUP: A = those
// chunks, B = a 128-column strip of the down matrix; epilogue scatters the fp32
// rows to partial[token][slot] (the unweighted down-partials of #129 "Scope").
template <bool GATEUP>
__global__ __launch_bounds__(256, 2) void grouped_gemm_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[2][STAGE_BYTES];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_tiles = min(a.tiles[0], a.tile_bound);
  const int nstrips = GATEUP ? max(a.F_pad, a.Fs_pad) / GU_COLS : a.d_pad / DN_COLS;
  if (n_tiles <= 0) return;
  // The valid workgroups (n_tiles * nstrips <= gridDim.x) are spread evenly
  // over the 8 XCDs, consecutive logical indices on the same XCD.
  const int n_valid = n_tiles * nstrips;
  const int per_xcd = (n_valid + 7) >> 3;
  const int slot = (int)blockIdx.x >> 3;
  if (slot >= per_xcd) return;
  const int blk = ((int)blockIdx.x & 7) * per_xcd + slot;
  if (blk >= n_valid) return;
  const int T = blk / nstrips, c = blk - (blk / nstrips) * nstrips;
  const int32_t* ent = a.tiles + 4 + 3 * T;
  const int g = ent[0], row0 = ent[1], row_end = ent[2];
  if (g < 0 || g >= a.G || row0 < 0 || row_end <= row0 || row_end > a.p_total) return;
  const bool shared = g >= a.E;
  const int Fg_pad = shared ? a.Fs_pad : a.F_pad;
  if (GATEUP && c >= Fg_pad / GU_COLS) return;
  const int KB = GATEUP ? a.d_pad / QB : Fg_pad / QB;
  const int KS = KB / KSTEP;
  const uint8_t* strip = GATEUP ? (shared ? a.sh_gu : a.gu + (size_t)g * a.gu_group)
                                : (shared ? a.sh_dn : a.dn + (size_t)g * a.dn_group);
  strip += (size_t)c * KS * KSTEP_BYTES;

  const int wrow0 = row0 + MT_WAVE * wave;  // first CSR row of this wavefront
  const bool active = wrow0 < row_end;
  const int t32 = T * (MT_WG / MT_WAVE) + wave;  // 32-row tile index of the h chunks
  const int8_t* ap;
  const uint16_t* asp;
  if (GATEUP) {
    const int p_lane = min(wrow0 + (lane & 31), row_end - 1);
    const int tok = min(max(a.tok_i[p_lane], 0), a.n_tokens - 1);
    ap = a.xq + (size_t)tok * a.d_pad + (lane >> 5) * 16;
    asp = a.xs + (size_t)tok * KB;
  } else {
    ap = a.hq + (size_t)t32 * a.kbmax * 1024 + lane * 16;
    asp = a.hs + ((size_t)t32 * 32 + (lane & 31)) * a.kbmax;
  }
  const size_t a_blk = GATEUP ? QB : 1024;  // bytes between consecutive blocks of one A row

  v16f acc[4];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) acc[tt] = (v16f){0};

  stage_kstep(strip, 0, ap, a_blk, lds[0], wave, lane);
  uint2 sa0 = make_uint2(0u, 0u), sa1 = make_uint2(0u, 0u);
  if (active) sa0 = *reinterpret_cast<const uint2*>(asp);
  // Unrolled by two so that each buffer and scale register is fixed.
  for (int ks = 0; ks < KS; ks += 2) {
    kloop_step(strip, ks, KS, ap, a_blk, asp, active, wave, lane, lds[0], lds[1], sa0, sa1, acc);
    if (ks + 1 < KS)
      kloop_step(strip, ks + 1, KS, ap, a_blk, asp, active, wave, lane, lds[1], lds[0], sa1, sa0, acc);
  }
  __syncthreads();  // every wavefront is out of the k loop: LDS is free for the epilogue
  if (!active) return;

  if (GATEUP) {
    // h = silu(gate) * up for the wavefront's 32 rows x 64 columns, transposed
    // through LDS ([32][65] floats, conflict-free) so that lane l then owns the
    // whole 32-block (row l%32, sub-strip l/32): amax, the two divisions and 32
    // codes per lane, written as two 16-byte pieces of the down GEMM's A chunk.
    float* hl = reinterpret_cast<float*>(&lds[0][0]) + wave * (32 * 65);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float gv = acc[sub][v], uv = acc[2 + sub][v];
        const float h = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
        hl[out_row(v, lane) * 65 + sub * 32 + (lane & 31)] = h;
      }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    const int r = lane & 31, sub = lane >> 5;
    float hv[32];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      hv[j] = hl[r * 65 + sub * 32 + j];
      amax = fmaxf(amax, fabsf(hv[j]));
    }
    uint32_t packed[8];
    uint16_t s16 = 0;
    if (amax == 0.0f) {
#pragma unroll
      for (int i = 0; i < 8; ++i) packed[i] = 0u;
    } else {
      const float id = 127.0f / amax;
      s16 = __half_as_ushort(__float2half_rn(amax / 127.0f));
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t w = 0u;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          float q = rintf(hv[4 * i + b] * id);
          q = fminf(fmaxf(q, -127.0f), 127.0f);
          w |= ((uint32_t)(int)q & 0xffu) << (8 * b);
        }
        packed[i] = w;
      }
    }
    const int kbf = 2 * c + sub;
    char* chunk = reinterpret_cast<char*>(a.hq) + ((size_t)t32 * a.kbmax + kbf) * 1024 + r * 16;
    *reinterpret_cast<uint4*>(chunk) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    *reinterpret_cast<uint4*>(chunk + 512) = make_uint4(packed[4], packed[5], packed[6], packed[7]);
    a.hs[((size_t)t32 * 32 + r) * a.kbmax + kbf] = s16;
  } else {
    const int p_lane = min(wrow0 + (lane & 31), row_end - 1);
    const int tok_l = a.tok_i[p_lane];
    const int slot_l = a.tok_k[p_lane];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = out_row(v, lane);
      const int tok = __shfl(tok_l, m, 64);
      const int slot = __shfl(slot_l, m, 64);
      if (wrow0 + m < row_end && (unsigned)tok < (unsigned)a.n_tokens && (unsigned)slot < (unsigned)a.kk) {
        float* dst = a.partial + ((size_t)tok * a.kk + slot) * a.d;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const int col = c * DN_COLS + tt * 32 + (lane & 31);
          if (col < a.d) dst[col] = acc[tt][v];
        }
      }
    }
  }
}

int grid_for(long wgs) { return (int)((wgs + 7) / 8 * 8); }

}  // namespace

hipError_t launch_gateup(const GemmArgs& a, hipStream_t s) {
  const long wgs = (long)a.tile_bound * (max(a.F_pad, a.Fs_pad) / GU_COLS);
  grouped_gemm_kernel<true><<<grid_for(wgs), 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_down(const GemmArgs& a, hipStream_t s) {
  const long wgs = (long)a.tile_bound * (a.d_pad / DN_COLS);
  grouped_gemm_kernel<false><<<grid_for(wgs), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
