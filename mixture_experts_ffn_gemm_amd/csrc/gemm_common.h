// gemm_common.h -- pieces shared by the grouped GEMM kernels of every weight
// format: operand types, the global->LDS copies and their waits, the
// pipeline-pinning anchors and the two epilogues (SwiGLU + requantise into
// the down GEMM's A operand; scatter of the down rows to the partials).
// Included by the GEMM sources only; everything here has internal linkage.
#pragma once

#include "internal.h"

namespace moe {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int NWAVE = MT_WG / MT_WAVE;                   // 4 wavefronts x 32 rows
constexpr int EPI_STRIDE = 65;                           // gate/up epilogue scratch row (floats)

__device__ inline int out_row(int v, int lane) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }

__device__ inline v4h as_v4h(uint32_t lo, uint32_t hi) {
  const uint2 u = make_uint2(lo, hi);
  return __builtin_bit_cast(v4h, u);
}
__device__ inline v4h as_v4h(uint2 u) { return __builtin_bit_cast(v4h, u); }

// global -> LDS copies: lane l moves `size` bytes from base + voff (base is
// wavefront-uniform, voff this lane's 32-bit offset) to LDS address
// m0 + size * l (m0 is wavefront-uniform).
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}

// Wait until at most n of this wavefront's copies are in flight (vector loads
// complete in order), then meet the other wavefronts.  The k-loop form also
// waits for this wavefront's LDS reads: operands of the buffer that the
// copies issued right after the barrier overwrite may still be in flight
// (their registers are consumed only after the barrier), and the barrier
// itself does not order them against other wavefronts' copies.
__device__ __forceinline__ void wait_copies_barrier_0() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
template <int N>
__device__ __forceinline__ void wait_copies_barrier_n() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait until at most N of this wavefront's copies are in flight and its LDS
// reads have returned, then meet the other wavefronts.
template <int N>
__device__ __forceinline__ void wait_copies_reads_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Copy sources of k-step 0: wavefront-uniform bases and per-lane 32-bit
// offsets.  K-step j adds j times the format's k-step bytes to the weight
// base.  Down reads h in slab form ([32 rows][128 B] per k-step): k-step j
// adds KSTEP chunks to the activation base and one k-step of scales (32 rows
// x KSTEP) to the scale base.  Gate/up gathers its code rows from the
// token-major codes gq[token][d_pad]: k-step j adds KSTEP blocks (128 bytes)
// to the base, and the per-lane offsets o_a name the tokens; its scales are
// in slab form like h's (gqs, per 32-row quarter of a tile).
struct Src {
  const uint8_t* w;    // the strip's first k-step
  const int8_t* a;     // gate/up: gq; down: this wavefront's h chunks
  const uint16_t* as;  // this wavefront's scale slab (gqs or hs)
  uint32_t o_w;        // 16 * lane: code chunk piece
  uint32_t o_ws;       // Q8_0: 16 KiB + 4 * lane + this wavefront's share of the weight scales
  uint32_t o_a[KSTEP]; // gate/up: chunk i's piece of this lane (see gather_offsets)
};

// The tokens of rows i0..i0+31 of tile T as the bucketing stored them
// (row_tok[T * 128 + i]; the tile's row i is CSR row row0 + i).  Scalar
// loads whose addresses depend only on T, so they can go out together with
// the tile's table entry, and waiting for them never waits for the copies in
// flight (those count on the vector-memory counter).  Entries past a group's
// rows were never written: gather_offsets discards them.
__device__ __forceinline__ void load_row_tokens(const GemmArgs& a, int T, int i0, int (&t)[MT_WAVE]) {
  typedef const int32_t __attribute__((address_space(4)))* tok_ptr;
  const tok_ptr p = (tok_ptr)a.row_tok + (size_t)T * MT_WG + i0;
#pragma unroll
  for (int m = 0; m < MT_WAVE; ++m) t[m] = p[m];
}

// Loads rows 32 wave and 32 wave + 16 of tile T's row tokens and waits for
// them, so that the two 64-byte scalar-cache lines of the wavefront's quarter
// of the tile are resident when the tile body reads them.
__device__ __forceinline__ void touch_row_tokens(const GemmArgs& a, int T, int wave) {
  typedef const int32_t __attribute__((address_space(4)))* tok_ptr;
  const tok_ptr p = (tok_ptr)a.row_tok + (size_t)T * MT_WG + MT_WAVE * wave;
  const int v = p[0] ^ p[16];
  asm volatile("" ::"s"(v));
}

// Gate/up copy offsets of the 32-row slab of rows i0..i0+31 of a tile whose
// rows are CSR rows row0..row_end-1, from their raw tokens t (a row past the
// end, or a token id out of range, reads token 0).  The LDS slab is
// [row][128 B] per k-step, the 16-byte piece p of row r at slot p ^ (r % 8);
// copy i of a k-step fills LDS bytes 1024 i + 16 lane, i.e. slot lane % 8 of
// row 8 i + lane / 8, so lane reads piece (lane % 8) ^ (lane / 8) -- bytes
// 16 p of the k-step's 128 -- of that row's token.  `chunk0` >= 0 asks for
// copy `chunk0` alone, in o_a[0] (the one-row-group pipeline, where each
// wavefront copies one chunk of a shared slab).
__device__ __forceinline__ void gather_offsets(const GemmArgs& a, const int (&raw)[MT_WAVE], int i0, int row0,
                                               int row_end, int lane, int chunk0, Src& s) {
  int t[MT_WAVE];
#pragma unroll
  for (int m = 0; m < MT_WAVE; ++m)
    t[m] = (row0 + i0 + m < row_end && (unsigned)raw[m] < (unsigned)a.n_tokens) ? raw[m] : 0;
  const int r8 = lane >> 3;
  const uint32_t piece = (uint32_t)(((lane & 7) ^ r8) << 4);
  const uint32_t dp = (uint32_t)a.d_pad;
  if (chunk0 >= 0) {
    int v = 0;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int u = chunk0 == 0 ? t[m] : chunk0 == 1 ? t[8 + m] : chunk0 == 2 ? t[16 + m] : t[24 + m];
      v = (r8 == m) ? u : v;
    }
    s.o_a[0] = (uint32_t)v * dp + piece;
  } else {
#pragma unroll
    for (int i = 0; i < KSTEP; ++i) {
      int v = t[8 * i];
#pragma unroll
      for (int m = 1; m < 8; ++m) v = (r8 == m) ? t[8 * i + m] : v;
      s.o_a[i] = (uint32_t)v * dp + piece;
    }
  }
}

// The activation copies of k-step j: chunk i of the slab (four per k-step),
// from the token-major codes (gate/up) or the h slab (down), and the slab's
// scales.
template <bool GATEUP>
__device__ __forceinline__ void dma_act_chunk(const Src& s, int j, int i, int lane, uint32_t lds) {
  if constexpr (GATEUP)
    dma16(s.a + (size_t)j * KSTEP * QB, s.o_a[i], lds);
  else
    dma16(s.a + ((size_t)j * KSTEP + i) * 1024, lane * 16, lds);
}
template <bool GATEUP>
__device__ __forceinline__ void dma_act_scales(const Src& s, int j, int lane, uint32_t lds) {
  dma4(s.as + (size_t)j * 32 * KSTEP, lane * 4, lds);
}

struct NoHook {
  __device__ void operator()(int) const {}
};

// Empty asm statements that take values "in and out" without emitting an
// instruction.  Volatile asm statements keep their order, so threading the
// pipeline's values through them pins the issue order of the MFMAs and the
// VALU groups (instruction selection would otherwise hoist all of a k-step's
// scale MFMAs, whose operands are known at its start, and run out of registers).
template <typename T>
__device__ __forceinline__ void anchor(T& v) {
  asm volatile("" : "+v"(v));
}
template <typename T, typename U>
__device__ __forceinline__ void anchor(T& v, U& u) {
  asm volatile("" : "+v"(v), "+v"(u));
}

// Per-wavefront constants of the pipelines: the accumulator input of every
// int8 MFMA (gate/up: the bits of 1.5 * 2^23; down: the bits of 1.5f), the
// constant A and B operands of the gate/up conversion MFMA (one non-zero K
// slot: -3072 * 4096 = -1.5 * 2^23) and, for down, the k-step's correction A
// operand.
struct Ctx {
  v16i magic;
  v4h sub_a, sub_b;
  v4h corr;
};

// The partial row [token][slot] of this lane's CSR row wrow0 + lane%32 (the
// down GEMM's destination), or -1 past the tile's rows or for a malformed pair.
__device__ __forceinline__ int partial_row(const GemmArgs& a, int lane, int wrow0, int row_end, int tok, int slt) {
  int ri = -1;
  if (wrow0 + (lane & 31) < row_end && (unsigned)tok < (unsigned)a.n_tokens && (unsigned)slt < (unsigned)a.kk)
    ri = tok * a.kk + slt;
  return ri;
}

// The down epilogue: the wavefront's 32 x 128 outputs scattered to the
// partial rows; ri is this lane's partial_row (lane r holds that of row r of
// the wavefront's 32).  All 16 exchanges are issued before any store.
__device__ __forceinline__ void epilogue_down(const GemmArgs& a, int lane, int cs, int g, int ri, v16f (&acc)[4]) {
  int rows[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) rows[v] = __shfl(ri, out_row(v, lane), 64);
  const bool full = (cs + 1) * DN_COLS <= a.d;  // the strip has no padding columns
  const int col0 = cs * DN_COLS + (lane & 31);
  // acc holds 2^-eg times the down product; scaled in place (pinned, so that
  // the scaling is not sunk into the conditional stores below)
  const int eg = __builtin_amdgcn_readfirstlane(a.dn_exp[g]);
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[tt][v] = ldexpf(acc[tt][v], eg);
    anchor(acc[tt]);
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    if (rows[v] >= 0) {
      float* dst = a.partial + (size_t)rows[v] * a.d + col0;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
        if (full || col0 + tt * 32 < a.d) dst[tt * 32] = acc[tt][v];
    }
  }
}

// The down epilogue through LDS: the wavefront's 32 x 128 outputs (scaled by
// 2^eg) transposed through its own [32][DN_EPI_STRIDE]-float area of the
// then idle stage buffers, so that each store writes two whole 512-byte rows
// of partials (16 stores per wavefront instead of 64 of 2 x 128 bytes).
// Every wavefront of the workgroup must be out of the k loop.  Rows 4 apart
// (the two lane halves of one accumulator register) start 32 banks apart.
constexpr int DN_EPI_STRIDE = 136;
__device__ __forceinline__ void epilogue_down_lds(const GemmArgs& a, char* lds, int lane, int wave, int cs, int g,
                                                  int ri, v16f (&acc)[4]) {
  const int eg = __builtin_amdgcn_readfirstlane(a.dn_exp[g]);
  float* el = reinterpret_cast<float*>(lds) + wave * (32 * DN_EPI_STRIDE);
#pragma unroll
  for (int tt = 0; tt < 4; ++tt)
#pragma unroll
    for (int v = 0; v < 16; ++v)
      el[out_row(v, lane) * DN_EPI_STRIDE + tt * 32 + (lane & 31)] = ldexpf(acc[tt][v], eg);
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  const int c4 = lane & 31, col = cs * DN_COLS + 4 * c4;
  const bool colok = col < a.d;  // d % 32 == 0: four columns are all inside or all padding
  int rr[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) rr[i] = __shfl(ri, 2 * i + (lane >> 5), 64);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = 2 * i + (lane >> 5);
    const float4 v = *reinterpret_cast<const float4*>(el + row * DN_EPI_STRIDE + 4 * c4);
    if (rr[i] >= 0 && colok) *reinterpret_cast<float4*>(a.partial + (size_t)rr[i] * a.d + col) = v;
  }
}

// Grouped GEMM.  GATEUP: A = the int8 token rows of the tile's (token, slot)
// pairs, which the quantiser wrote in chunk form at their padded rows; B = the
// [gate;up] strip of 64 SwiGLU columns; epilogue h = silu(gate) * up,
// requantised per 32 into the down GEMM's A-operand chunks.  !GATEUP: A = those
// chunks, B = a 128-column strip of the down matrix; epilogue scatters the fp32
// rows to partial[token][slot] (the unweighted down-partials of #129 "Scope").
//
// The epilogue of one wavefront's 32 rows (CSR rows wrow0.., 32-row tile
// t32) against strip cs of group g; tok / slt are this lane's (token, slot)
// for down.  Gate/up uses this wavefront's area at the start of the LDS.
// DN_LDS: the down epilogue through LDS (epilogue_down_lds; the caller's LDS
// must hold NWAVE x 32 x DN_EPI_STRIDE floats), else direct scattered stores.
template <bool GATEUP, bool DN_LDS = false>
__device__ __forceinline__ void epilogue(const GemmArgs& a, char* lds, int lane, int wave, int t32, int cs, int g,
                                         int wrow0, int row_end, int tok, int slt, v16f (&acc)[4]) {
  if constexpr (GATEUP) {
    // h = silu(gate) * up for the wavefront's 32 rows x 64 columns, transposed
    // through LDS ([32][65] floats, conflict-free) so that lane l then owns the
    // whole 32-block (row l%32, sub-strip l/32): amax, the two divisions and 32
    // codes per lane, written as two 16-byte pieces of the down GEMM's A chunk.
    float* hl = reinterpret_cast<float*>(lds) + wave * (32 * EPI_STRIDE);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float gv = acc[sub][v], uv = acc[2 + sub][v];
        const float h = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
        hl[out_row(v, lane) * EPI_STRIDE + sub * 32 + (lane & 31)] = h;
      }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    const int r = lane & 31, sub = lane >> 5;
    float hv[32];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      hv[j] = hl[r * EPI_STRIDE + sub * 32 + j];
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
    // block kbf of h = pieces 2(kbf%4), +1 of k-step kbf/4 in row r's line
    const int kbf = 2 * cs + sub, p0 = 2 * (kbf & 3);
    char* line = reinterpret_cast<char*>(a.hq) +
                 (((size_t)t32 * (a.kbmax / KSTEP) + (kbf >> 2)) * 32 + r) * 128;
    *reinterpret_cast<uint4*>(line + ((p0 ^ (r & 7)) << 4)) =
        make_uint4(packed[0], packed[1], packed[2], packed[3]);
    *reinterpret_cast<uint4*>(line + (((p0 + 1) ^ (r & 7)) << 4)) =
        make_uint4(packed[4], packed[5], packed[6], packed[7]);
    a.hs[(((size_t)t32 * (a.kbmax / KSTEP) + (kbf >> 2)) * 32 + r) * KSTEP + (kbf & 3)] = s16;
  } else if constexpr (DN_LDS) {
    epilogue_down_lds(a, lds, lane, wave, cs, g, partial_row(a, lane, wrow0, row_end, tok, slt), acc);
  } else {
    epilogue_down(a, lane, cs, g, partial_row(a, lane, wrow0, row_end, tok, slt), acc);
  }
}

// The partial accumulators of a split row group, summed into its first
// wavefront (si = 0) in the fixed order ((p0 + p1) + p2) + p3 through the
// (then idle) stage buffers.  Every wavefront of the workgroup calls this.
__device__ __forceinline__ void split_reduce(char* lds, int S, int rg, int si, int lane, v16f (&acc)[4]) {
  __syncthreads();  // every wavefront is out of the k loop: the stage buffers are free
  float* red = reinterpret_cast<float*>(lds);
  if (si > 0) {
    float* dst = red + (size_t)(rg * (S - 1) + si - 1) * 64 * 64;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) dst[(t * 16 + v) * 64 + lane] = acc[t][v];
  }
  __syncthreads();
  if (si == 0) {
    for (int p = 1; p < S; ++p) {
      const float* src = red + (size_t)(rg * (S - 1) + p - 1) * 64 * 64;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[t][v] = acc[t][v] + src[(t * 16 + v) * 64 + lane];
    }
  }
  __syncthreads();  // the reduction buffers are read before any epilogue reuses the LDS
}

inline int grid_for(long wgs) { return (int)((wgs + 7) / 8 * 8); }

}  // namespace
}  // namespace moe
