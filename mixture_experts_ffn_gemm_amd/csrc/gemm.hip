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
// Arithmetic per 32-block, per 32x32 output tile of a wavefront, gate/up:
//   v_mfma_i32_32x32x32_i8  -> exact int32 block sums C[m][n]
//   v_mfma_f32_32x32x8_f16  -> S[m][n] = sa[m] * sw[n]: an outer product of the
//                              two binary16 block scales, exact in fp32 (only
//                              one of the 8 K slots is non-zero in A),
// then the VALU does acc = fma(float(C), S, acc): two VALU operations per
// output element per block, which bounds the kernel.  Gate/up keeps this exact
// form because its output is requantised (a value moved across a rounding
// boundary of the h quantiser changes a code).
//
// Down (its fp32 output is final): the int8 MFMA's accumulator input is the
// bit pattern of 1.5f, so its int32 result, read as a float, is exactly
// D = 1.5 + C * 2^-23 (|C| < 2^19 leaves the exponent field alone).  With the
// weight scales stored as W = sw * 2^(23-e) the scale MFMA gives
// S = sa * W = 2^(23-e) * sa * sw, and one VALU fma per element and block,
// acc = fma(D, S, acc), adds 2^-e * C * sa * sw + 1.5 * S.  Once per k-step
// a third MFMA takes the accumulator as its input and subtracts the 4 blocks'
// 1.5 * S (A = -sa twice, B = {W, W/2} per block).  The epilogue multiplies
// by 2^e.  The only rounding beyond the exact form is that of the corrected
// accumulator, whose magnitude is that of the 1.5 * S terms: about 1e-4
// relative to the output, well inside the output tolerance.
//
// * Memory: per k-step (4 blocks) a workgroup stages the strip's weight codes
//   (16 chunks of 1 KiB: [block][tile]) and scales (1 KiB; 2 KiB of pairs for
//   down), and each
//   wavefront its 32 activation rows (a 4 KiB slab [row][128 B], the 16-byte
//   pieces of row r XOR-swizzled by r%8 so that the MFMA operand reads are
//   free of LDS bank conflicts) and their scales (256 B), with direct
//   global->LDS copies into one of two LDS buffers.  Every copy reads whole
//   cache lines: gate/up gathers its rows from the token-major codes, each
//   copy covering 8 rows' 128-byte k-step pieces (a copy of 32 rows' 32-byte
//   blocks would hold one vector-L1 miss slot per row), and reads their
//   scales, which the quantiser stores per expert slot, in slab form; down
//   reads h and its scales, which the gate/up epilogue stores in slab form.
//   Every wavefront issues
//   exactly Lay::DMA copies per k-step, in two halves (weights right after
//   the barrier, activations one block later) so that the copies of all
//   wavefronts never queue at once.  The copies are inline assembly, so the
//   compiler never inserts its own (conservative) waits for them, and they are
//   waited for with explicit vmcnt counts (the loop issues no other
//   vector-memory instructions).
// * One barrier per k-step, before the last block of k-step j: it publishes
//   k-step j+1 (copied four blocks earlier) and proves that every wavefront
//   has read all of k-step j, whose buffer then receives k-step j+2.
// * LDS operands are read one block ahead: the A chunk and the 4 B chunks of
//   block b+1 are requested before block b is computed, so LDS latency and
//   bandwidth overlap the MFMA/VALU work instead of stalling after a barrier.
// * Within a block the 4 tiles are software-pipelined one step deep with the
//   issue order pinned (gate/up: MFMA(t+1), convert(t), scale MFMA(t+1),
//   accumulate(t); down: MFMA(t+1), accumulate(t) half 1, scale MFMA(t+1),
//   accumulate(t) half 2), and the
//   pipeline runs on across blocks and k-steps.
// Operand layouts (gfx950): A lane l = row l%32, bytes/halves k = 16*(l/32)+j
// (i8) or 4*(l/32)+j (f16x8); B likewise by column; D lane l = column l%32,
// register v = row 8*(v/4) + 4*(l/32) + v%4.
#include <type_traits>

#include "device_util.h"
#include "gemm_common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int B_OFF = 0;                                 // weight codes [block][tile] x 1 KiB
constexpr int BS_OFF = 16 * 1024;                        // weight scales (gate/up: [tile][32 rows][4
                                                         // blocks]; down: [tile][half][32 rows][4])

// Stage layout of one k-step buffer: the weight k-step (17 or 18 KiB), then
// the activation chunks [wave][block] x 1 KiB and their scales [wave][32 rows][4 blocks].
template <bool GATEUP>
struct Lay {
  static constexpr int W_BYTES = GATEUP ? KSTEP_BYTES : DN_KSTEP_BYTES;
  static constexpr int A_OFF = W_BYTES;
  static constexpr int AS_OFF = A_OFF + NWAVE * KSTEP * 1024;
  static constexpr int STAGE = AS_OFF + NWAVE * 32 * KSTEP * 2;  // 34 / 35 KiB
  static constexpr int DMA = GATEUP ? 10 : 11;                   // copies per wavefront per k-step
};
static_assert(NWAVE * 32 * EPI_STRIDE * 4 <= Lay<true>::STAGE, "epilogue scratch must fit in one buffer");
static_assert(2 * 2 * Lay<false>::STAGE <= 160 * 1024, "two workgroups per CU must fit in the LDS");
static_assert(NWAVE * 32 * DN_EPI_STRIDE * 4 <= 2 * Lay<false>::STAGE, "the down epilogue's transpose must fit in the stage buffers");

// This wavefront's copies of k-step j into the buffer at LDS address L, in
// two halves issued at different points of the k loop, so that the copies of
// all wavefronts never queue at once: the weight half (code chunks wave + 4i
// and a quarter of the weight scales) and the activation half (its 4
// activation chunks and its 32 rows' activation scales).
template <bool GATEUP>
__device__ __forceinline__ void issue_weights(const Src& s, int j, uint32_t L, int wave) {
  const uint8_t* w = s.w + (size_t)j * Lay<GATEUP>::W_BYTES;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = wave + 4 * i;
    dma16(w + c * 1024, s.o_w, L + B_OFF + c * 1024);
  }
  if (GATEUP) {
    dma4(w, s.o_ws, L + BS_OFF + wave * 256);
  } else {
    dma4(w, s.o_ws, L + BS_OFF + wave * 512);
    dma4(w, s.o_ws + 256, L + BS_OFF + wave * 512 + 256);
  }
}
template <bool GATEUP>
__device__ __forceinline__ void issue_acts(const Src& s, int j, uint32_t L, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < KSTEP; ++i)
    dma_act_chunk<GATEUP>(s, j, i, lane, L + Lay<GATEUP>::A_OFF + (wave * KSTEP + i) * 1024);
  dma_act_scales<GATEUP>(s, j, lane, L + Lay<GATEUP>::AS_OFF + wave * 256);
}

// The same copies issued in parts, one part per tile of a block (the hook
// of compute_block calls part t right after tile t's int8 MFMA), so that a
// wavefront's copies go out between matrix instructions instead of in one
// burst that stalls its issue: parts 0 and 1 two 1 KiB chunks each, part 2
// the scales, part 3 nothing.
template <bool GATEUP>
__device__ __forceinline__ void issue_weights_part(const Src& s, int j, uint32_t L, int wave, int p) {
  const uint8_t* w = s.w + (size_t)j * Lay<GATEUP>::W_BYTES;
  if (p < 2) {
#pragma unroll
    for (int i = 2 * p; i < 2 * p + 2; ++i) {
      const int c = wave + 4 * i;
      dma16(w + c * 1024, s.o_w, L + B_OFF + c * 1024);
    }
  } else if (p == 2) {
    if (GATEUP) {
      dma4(w, s.o_ws, L + BS_OFF + wave * 256);
    } else {
      dma4(w, s.o_ws, L + BS_OFF + wave * 512);
      dma4(w, s.o_ws + 256, L + BS_OFF + wave * 512 + 256);
    }
  }
}
template <bool GATEUP>
__device__ __forceinline__ void issue_acts_part(const Src& s, int j, uint32_t L, int wave, int lane, int p) {
  if (p < 2) {
#pragma unroll
    for (int i = 2 * p; i < 2 * p + 2; ++i)
      dma_act_chunk<GATEUP>(s, j, i, lane, L + Lay<GATEUP>::A_OFF + (wave * KSTEP + i) * 1024);
  } else if (p == 2) {
    dma_act_scales<GATEUP>(s, j, lane, L + Lay<GATEUP>::AS_OFF + wave * 256);
  }
}

// Register operands of one block: this wavefront's A chunk and the 4 B chunks.
struct Ops {
  v4i a;
  v4i b[4];
};

// a_off: LDS offset of the 32-row activation slab within the stage buffer.
__device__ __forceinline__ void read_block_at(const char* buf, int a_off, int b, int lane, Ops& o) {
  // A: row lane%32, piece 2b + lane/32 of the k-step, stored at its row's
  // 128-byte line position (piece ^ row%8)
  const int r = lane & 31, p = 2 * b + (lane >> 5);
  o.a = *reinterpret_cast<const v4i*>(buf + a_off + r * 128 + ((p ^ (r & 7)) << 4));
#pragma unroll
  for (int t = 0; t < 4; ++t)
    o.b[t] = *reinterpret_cast<const v4i*>(buf + B_OFF + (b * 4 + t) * 1024 + lane * 16);
}
template <bool GATEUP>
__device__ __forceinline__ void read_block(const char* buf, int b, int wave, int lane, Ops& o) {
  read_block_at(buf, Lay<GATEUP>::A_OFF + wave * (KSTEP * 1024), b, lane, o);
}

// Gate/up: the k-step's weight scales of the 4 tiles (column lane%32, blocks
// 0-3: the B operands of the scale MFMA) and the activation scales of this
// lane's row (lanes 32-63 supply the zero K slots 4-7).
struct GuScales {
  v4h sw[4];
  uint2 sa;
};

// as_off: LDS offset of the slab's activation scales within the stage buffer.
__device__ __forceinline__ void read_scales_at(const char* buf, int as_off, int lane, GuScales& s) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint2 p = *reinterpret_cast<const uint2*>(buf + BS_OFF + (t * 32 + (lane & 31)) * 8);
    s.sw[t] = as_v4h(p.x, p.y);
  }
  const uint2 p = *reinterpret_cast<const uint2*>(buf + as_off + (lane & 31) * 8);
  const uint32_t m = lane < 32 ? 0xffffffffu : 0u;
  s.sa = make_uint2(p.x & m, p.y & m);
}

// A operand of the scale MFMA for block b: K slot b holds this row's scale.
__device__ __forceinline__ v4h sa_slot(const uint2 sa, int b) {
  const uint32_t m = (b & 1) ? 0xffff0000u : 0x0000ffffu;
  return b < 2 ? as_v4h(sa.x & m, 0u) : as_v4h(0u, sa.y & m);
}

// Down: per tile the B operand shared by the scale and correction MFMAs (lane
// l: column l%32, K slots 4(l/32)..4(l/32)+3 = {W, W/2} of blocks 2(l/32) and
// 2(l/32)+1), and this lane's pair of activation scales q (row l%32, the same
// two blocks).
struct DnScales {
  uint2 wb[4];
  uint32_t q;
};

__device__ __forceinline__ void read_scales_at(const char* buf, int as_off, int lane, DnScales& s) {
#pragma unroll
  for (int t = 0; t < 4; ++t) s.wb[t] = *reinterpret_cast<const uint2*>(buf + BS_OFF + t * 512 + lane * 8);
  const uint2 p = *reinterpret_cast<const uint2*>(buf + as_off + (lane & 31) * 8);
  s.q = lane < 32 ? p.x : p.y;
}

template <typename SC>
__device__ __forceinline__ void read_scales(const char* buf, int wave, int lane, SC& s) {
  constexpr bool GATEUP = std::is_same<SC, GuScales>::value;
  read_scales_at(buf, Lay<GATEUP>::AS_OFF + wave * 256, lane, s);
}

// A operand of the down scale MFMA for block b: K slot 2b (the slot whose B
// entry is W of block b) holds this row's activation scale.
__device__ __forceinline__ v4h dn_sa_slot(uint32_t q, int b, int lane) {
  const uint32_t v = ((lane >> 5) == (b >> 1)) ? q : 0u;
  return (b & 1) ? as_v4h(0u, v >> 16) : as_v4h(v & 0xffffu, 0u);
}

// A operand of the correction MFMA: -sa in both slots of each block, so that
// A.B = -(sa W + sa W/2) = -1.5 S summed over the k-step's 4 blocks.
__device__ __forceinline__ v4h dn_corr_a(uint32_t q) {
  const uint32_t lo = q & 0xffffu, hi = q >> 16;
  return as_v4h((lo | (lo << 16)) ^ 0x80008000u, (hi | (hi << 16)) ^ 0x80008000u);
}

// One block (4 tiles) of the gate/up pipeline, which runs two tiles ahead.
// On entry dn holds the int8 MFMA of tile 1 of this block (as the float
// 1.5 * 2^23 + C), cf = float(C) and s the scale product of tile 0; on exit
// the same for the next block (operands `on`, scales `sn`, block bn).  Per
// tile t: int8 MFMA(t+2), a third of acc(t) = fma(cf(t), s(t), acc(t)), the
// conversion MFMA(t+1) (C input dn, minus 1.5 * 2^23: exactly float(C)), a
// third, scale MFMA(t+1), the last third.  The VALU does one fma per element
// and block; the conversion runs on the matrix pipe, and the result is the
// same as fma(float(C), S, acc).
template <typename H = NoHook>
__device__ __forceinline__ void compute_block(const Ops& o, const GuScales& sc, int b, const Ops& on,
                                              const GuScales& sn, int bn, bool, const Ctx& cx, int,
                                              v16i& dn, v16f& cf, v16f& s, v16f (&acc)[4], const H& hook = H()) {
  const v16f zf = {0};
  v4h sav = sa_slot(sc.sa, b);
  v4h savn = sa_slot(sn.sa, bn);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    v16i dnn = t < 2 ? __builtin_amdgcn_mfma_i32_32x32x32_i8(o.a, o.b[t + 2], cx.magic, 0, 0, 0)
                     : __builtin_amdgcn_mfma_i32_32x32x32_i8(on.a, on.b[t - 2], cx.magic, 0, 0, 0);
    anchor(dnn, dn);
    hook(t);
#pragma unroll
    for (int v = 0; v < 5; ++v) acc[t][v] = __builtin_fmaf(cf[v], s[v], acc[t][v]);
    anchor(acc[t]);
    v16f cfn = __builtin_amdgcn_mfma_f32_32x32x8f16(cx.sub_a, cx.sub_b, __builtin_bit_cast(v16f, dn), 0, 0, 0);
    anchor(cfn, acc[t]);
#pragma unroll
    for (int v = 5; v < 10; ++v) acc[t][v] = __builtin_fmaf(cf[v], s[v], acc[t][v]);
    if (t < 3)
      anchor(acc[t], sav);
    else
      anchor(acc[t], savn);
    v16f sx = t < 3 ? __builtin_amdgcn_mfma_f32_32x32x8f16(sav, sc.sw[t + 1], zf, 0, 0, 0)
                    : __builtin_amdgcn_mfma_f32_32x32x8f16(savn, sn.sw[0], zf, 0, 0, 0);
    anchor(sx, acc[t]);
#pragma unroll
    for (int v = 10; v < 16; ++v) acc[t][v] = __builtin_fmaf(cf[v], s[v], acc[t][v]);
    anchor(acc[t]);
    dn = dnn;
    cf = cfn;
    s = sx;
  }
}

// One block of the down pipeline.  Per tile t: int8 MFMA(t+1) from the 1.5f
// bias, half of acc(t) = fma(D(t), S(t), acc(t)), scale MFMA(t+1), the other
// half; after the wavefront's last block of the k-step (corr) the correction
// MFMA subtracts the 1.5 * S terms of the k-step's blocks it computed.
template <typename H = NoHook>
__device__ __forceinline__ void compute_block(const Ops& o, const DnScales& sc, int b, const Ops& on,
                                              const DnScales& sn, int bn, bool corr, const Ctx& cx,
                                              int lane, v16i& c, v16f&, v16f& s, v16f (&acc)[4],
                                              const H& hook = H()) {
  const v16f zf = {0};
  v4h sav = dn_sa_slot(sc.q, b, lane);
  v4h savn = dn_sa_slot(sn.q, bn, lane);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    // Each MFMA is followed by 8 fmas (32 cycles), the time it occupies the
    // matrix pipe, so that neither MFMA waits at issue for the other.
    v16i cn = t < 3 ? __builtin_amdgcn_mfma_i32_32x32x32_i8(o.a, o.b[t + 1], cx.magic, 0, 0, 0)
                    : __builtin_amdgcn_mfma_i32_32x32x32_i8(on.a, on.b[0], cx.magic, 0, 0, 0);
    anchor(cn, c);
    hook(t);
    const v16f d = __builtin_bit_cast(v16f, c);
#pragma unroll
    for (int v = 0; v < 8; ++v) acc[t][v] = __builtin_fmaf(d[v], s[v], acc[t][v]);
    if (t < 3)
      anchor(acc[t], sav);
    else
      anchor(acc[t], savn);
    v16f sx = t < 3 ? __builtin_amdgcn_mfma_f32_32x32x8f16(sav, as_v4h(sc.wb[t + 1]), zf, 0, 0, 0)
                    : __builtin_amdgcn_mfma_f32_32x32x8f16(savn, as_v4h(sn.wb[0]), zf, 0, 0, 0);
    anchor(sx, acc[t]);
#pragma unroll
    for (int v = 8; v < 16; ++v) acc[t][v] = __builtin_fmaf(d[v], s[v], acc[t][v]);
    anchor(acc[t]);
    if (corr) {
      acc[t] = __builtin_amdgcn_mfma_f32_32x32x8f16(cx.corr, as_v4h(sc.wb[t]), acc[t], 0, 0, 0);
      anchor(acc[t]);
    }
    c = cn;
    s = sx;
  }
}

template <bool GATEUP>
using ScalesT = typename std::conditional<GATEUP, GuScales, DnScales>::type;

// K-step j of an active wavefront, from buffer `cur`; k-step j+1 is (or, for
// the last k-step, stale data standing in for it is) in `nxt`.  On entry X
// holds block 0's operands, sc the k-step's scales and c/cf/s the pipeline
// state of (block 0, tile 0); on exit X, sn and c/cf/s are those of k-step
// j+1 (after the last k-step they belong to no k-step and are discarded).
template <bool GATEUP>
__device__ __forceinline__ void kstep(const Src& src, int j, int KS, int wave, int lane, const char* cur,
                                      const char* nxt, uint32_t cur_lds, uint32_t nxt_lds, Ops& X,
                                      Ops& Y, const ScalesT<GATEUP>& sc, ScalesT<GATEUP>& sn,
                                      Ctx& cx, v16i& c, v16f& cf, v16f& s, v16f (&acc)[4]) {
  // The activation half of k-step j+1 goes out during block 0 (its weight
  // half during block 3 of k-step j-1; k-steps 0 and 1 are copied whole by
  // the prologue).
  const bool acts = j >= 1 && j + 1 < KS;
  if constexpr (!GATEUP) cx.corr = dn_corr_a(sc.q);
  read_block<GATEUP>(cur, 1, wave, lane, Y);
  compute_block(X, sc, 0, Y, sc, 1, false, cx, lane, c, cf, s, acc, [&](int t) {
    if (acts) issue_acts_part<GATEUP>(src, j + 1, nxt_lds, wave, lane, t);
  });
  read_block<GATEUP>(cur, 2, wave, lane, X);
  compute_block(Y, sc, 1, X, sc, 2, false, cx, lane, c, cf, s, acc);
  read_block<GATEUP>(cur, 3, wave, lane, Y);
  compute_block(X, sc, 2, Y, sc, 3, false, cx, lane, c, cf, s, acc);
  // k-step j+1 has landed for every wavefront, and every wavefront has read
  // all of k-step j: its buffer takes k-step j+2 (the weight half, during
  // block 3).
  if (j + 1 < KS) wait_copies_barrier_0();
  const bool weights = j + 2 < KS;
  read_block<GATEUP>(nxt, 0, wave, lane, X);
  read_scales(nxt, wave, lane, sn);
  compute_block(Y, sc, 3, X, sn, 0, true, cx, lane, c, cf, s, acc, [&](int t) {
    if (weights) issue_weights_part<GATEUP>(src, j + 2, cur_lds, wave, t);
  });
}

// Split-K: the correction operand of the blocks a split wavefront computes
// (S = 4: block si; S = 2: blocks si and si + 2).  Lane half h holds the
// slots of blocks 2h and 2h + 1; the slots of blocks left to other
// wavefronts are zeroed, so their (never added) 1.5 * S terms are not
// subtracted either.
template <int S>
__device__ __forceinline__ v4h dn_corr_split(uint32_t q, int lane, int si) {
  const int h = lane >> 5;
  const bool keep_lo = (S == 4) ? (2 * h == si) : (si == 0);
  const bool keep_hi = (S == 4) ? (2 * h + 1 == si) : (si == 1);
  return dn_corr_a(q & ((keep_lo ? 0x0000ffffu : 0u) | (keep_hi ? 0xffff0000u : 0u)));
}

// K-step j of a split-K wavefront of a two-row-group tile (SharpInference
// #406 "References": the split-K int8 GEMM follow-up).  A tile whose rows
// fill only two of the four 32-row wavefront slots would leave two
// wavefronts idle; instead the two wavefronts of each row group share its
// blocks: wavefront si computes blocks si and si + 2 of every k-step into its
// own partial accumulators, which the kernel sums in a fixed order at the
// end.  Copies, barriers and their placement are those of kstep (every
// wavefront meets the same barriers and issues the same copies; each copies
// its row group's activation slab into its own LDS area).  On entry X holds
// block si of k-step j; on exit the same for k-step j+1.
template <bool GATEUP>
__device__ __forceinline__ void kstep_split2(const Src& src, int j, int KS, int wave, int lane, int si,
                                             const char* cur, const char* nxt, uint32_t cur_lds,
                                             uint32_t nxt_lds, Ops& X, Ops& Y, const ScalesT<GATEUP>& sc,
                                             ScalesT<GATEUP>& sn, Ctx& cx, v16i& c, v16f& cf, v16f& s,
                                             v16f (&acc)[4]) {
  const bool acts = j >= 1 && j + 1 < KS;
  if constexpr (!GATEUP) cx.corr = dn_corr_split<2>(sc.q, lane, si);
  read_block<GATEUP>(cur, si + 2, wave, lane, Y);
  compute_block(X, sc, si, Y, sc, si + 2, false, cx, lane, c, cf, s, acc, [&](int t) {
    if (acts) issue_acts_part<GATEUP>(src, j + 1, nxt_lds, wave, lane, t);
  });
  if (j + 1 < KS) wait_copies_barrier_0();
  const bool weights = j + 2 < KS;
  read_block<GATEUP>(nxt, si, wave, lane, X);
  read_scales(nxt, wave, lane, sn);
  compute_block(Y, sc, si + 2, X, sn, si, true, cx, lane, c, cf, s, acc, [&](int t) {
    if (weights) issue_weights_part<GATEUP>(src, j + 2, cur_lds, wave, t);
  });
}

// One-row-group tiles (at most 32 rows): the four wavefronts split every
// k-step, wavefront si computing block si.  Each wavefront then does a
// quarter of a full tile's matrix work per k-step while the workgroup still
// stages the whole weight k-step, so the k loop is bound by the latency of
// the global->LDS copies rather than by the matrix pipe.  This pipeline
// therefore keeps three k-steps in LDS instead of two (a stage holds the
// weight k-step and the single activation slab) and issues the copies of
// k-step j+3 at the barrier of k-step j, two k-steps earlier than they are
// needed.
template <bool GATEUP>
struct Lay1 {
  static constexpr int A_OFF = Lay<GATEUP>::W_BYTES;      // the slab's 4 chunks [row][128 B]
  static constexpr int AS_OFF = A_OFF + KSTEP * 1024;     // their scales [32 rows][4 blocks]
  static constexpr int STAGE = AS_OFF + 32 * KSTEP * 2;   // 21.25 / 22.25 KiB
  static constexpr int DMA = Lay<GATEUP>::DMA - KSTEP + 1;  // copies per wavefront per k-step
};
static_assert(3 * Lay1<true>::STAGE <= 2 * Lay<true>::STAGE, "three stages must fit in the LDS buffers");
static_assert(3 * Lay1<false>::STAGE <= 2 * Lay<false>::STAGE, "three stages must fit in the LDS buffers");
static_assert(Lay1<true>::STAGE % 256 == 0 && Lay1<false>::STAGE % 256 == 0, "stage alignment");

// This wavefront's copies of k-step j into the stage at LDS address L: its
// share of the weight k-step, activation chunk `wave` of the slab, and the
// slab's scales (every wavefront copies the same 256 bytes, so that all issue
// the same number of copies).
template <bool GATEUP>
__device__ __forceinline__ void issue_kstep1(const Src& s, int j, uint32_t L, int wave, int lane) {
  issue_weights<GATEUP>(s, j, L, wave);
  if constexpr (GATEUP)
    dma_act_chunk<true>(s, j, 0, lane, L + Lay1<GATEUP>::A_OFF + wave * 1024);
  else
    dma_act_chunk<false>(s, j, wave, lane, L + Lay1<GATEUP>::A_OFF + wave * 1024);
  dma_act_scales<GATEUP>(s, j, lane, L + Lay1<GATEUP>::AS_OFF);
}

// K-step j of a one-row-group tile.  On entry X and sc hold block si of
// k-step j (read from its stage in the previous k-step); k-steps j+1 and j+2
// are in flight.  The barrier publishes k-step j+1 and proves that every
// wavefront has read k-step j, whose stage then receives k-step j+3.  On exit
// Y and sn hold block si of k-step j+1 (stale data after the last k-step,
// never used).
template <bool GATEUP>
__device__ __forceinline__ void kstep1(const Src& src, int j, int KS, int wave, int lane, int si,
                                       const char* lds, uint32_t lds_base, const Ops& X, Ops& Y,
                                       const ScalesT<GATEUP>& sc, ScalesT<GATEUP>& sn, Ctx& cx, v16i& c,
                                       v16f& cf, v16f& s, v16f (&acc)[4]) {
  using L1 = Lay1<GATEUP>;
  if constexpr (!GATEUP) cx.corr = dn_corr_split<4>(sc.q, lane, si);
  const int st = j % 3;
  const int sn1 = st == 2 ? 0 : st + 1;
  if (j + 1 < KS) {
    if (j + 2 < KS)
      wait_copies_reads_barrier<L1::DMA>();
    else
      wait_copies_reads_barrier<0>();
    if (j + 3 < KS) issue_kstep1<GATEUP>(src, j + 3, lds_base + st * L1::STAGE, wave, lane);
  }
  const char* nb = lds + sn1 * L1::STAGE;
  read_block_at(nb, L1::A_OFF, si, lane, Y);
  read_scales_at(nb, L1::AS_OFF, lane, sn);
  compute_block(X, sc, si, Y, sn, si, true, cx, lane, c, cf, s, acc);
}

// Pipeline constants and the state of (block si, tile 0) from the first
// block's operands X and scales s0: for gate/up the int8 MFMA of tile 1,
// float(C) and the scale product of tile 0; for down the int8 MFMA and the
// scale product of tile 0.
template <bool GATEUP>
__device__ __forceinline__ void pipeline_init(const Ops& X, const ScalesT<GATEUP>& s0, int si, int lane, Ctx& cx,
                                              v16i& c, v16f& cf, v16f& s) {
  const v16f zf = {0};
  if constexpr (GATEUP) {
#pragma unroll
    for (int v = 0; v < 16; ++v) cx.magic[v] = 0x4b400000;  // 1.5 * 2^23
    anchor(cx.magic);  // one register copy, never rematerialised
    const _Float16 h0 = 0;
    cx.sub_a = lane < 32 ? (v4h){(_Float16)-3072.0f, h0, h0, h0} : (v4h){h0, h0, h0, h0};
    cx.sub_b = lane < 32 ? (v4h){(_Float16)4096.0f, h0, h0, h0} : (v4h){h0, h0, h0, h0};
    anchor(cx.sub_a, cx.sub_b);
    const v16i d0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(X.a, X.b[0], cx.magic, 0, 0, 0);
    c = __builtin_amdgcn_mfma_i32_32x32x32_i8(X.a, X.b[1], cx.magic, 0, 0, 0);
    cf = __builtin_amdgcn_mfma_f32_32x32x8f16(cx.sub_a, cx.sub_b, __builtin_bit_cast(v16f, d0), 0, 0, 0);
    s = __builtin_amdgcn_mfma_f32_32x32x8f16(sa_slot(s0.sa, si), s0.sw[0], zf, 0, 0, 0);
  } else {
#pragma unroll
    for (int v = 0; v < 16; ++v) cx.magic[v] = 0x3fc00000;  // 1.5f
    anchor(cx.magic);
    c = __builtin_amdgcn_mfma_i32_32x32x32_i8(X.a, X.b[0], cx.magic, 0, 0, 0);
    s = __builtin_amdgcn_mfma_f32_32x32x8f16(dn_sa_slot(s0.q, si, lane), as_v4h(s0.wb[0]), zf, 0, 0, 0);
  }
}

// The work of one (tile, strip) workgroup whose tile has three or four
// 32-row groups (S = 1: one row group per wavefront) or two (S = 2: see
// kstep_split2).  Each split factor is a separate, self-contained body
// (nothing it computes is live across the others), so that each gets its own
// register allocation.
template <bool GATEUP, int S>
__device__ __forceinline__ void tile_work(const GemmArgs& a, char (&lds)[2][Lay<GATEUP>::STAGE], int lane,
                                          int wave, int T, int cs, int g, int row0, int row_end, int KS,
                                          const uint8_t* strip) {
  static_assert(S == 1 || S == 2, "split factors of tile_work");
  using L = Lay<GATEUP>;
  const int rg = wave / S, si = wave - rg * S;
  const int wrow0 = row0 + MT_WAVE * rg;    // first CSR row of this wavefront's row group
  const bool active = wrow0 < row_end;      // wavefront-uniform (every wavefront when S > 1)
  const int t32 = T * NWAVE + rg;           // 32-row tile index of the A slab and the h chunks
  // A operand: gate/up gathers the 32 rows of its row group from the
  // token-major codes; down reads the h slab of 32-row quarter t32 of the tile.
  Src src;
  src.w = strip;
  src.o_w = lane * 16;
  src.o_ws = 16 * 1024 + wave * (GATEUP ? 256 : 512) + lane * 4;
  if constexpr (GATEUP) {
    src.a = a.gq;
    src.as = a.gqs + (size_t)t32 * (a.d_pad / QB) * 32;
    int t[MT_WAVE];
    load_row_tokens(a, T, MT_WAVE * rg, t);
    gather_offsets(a, t, MT_WAVE * rg, row0, row_end, lane, -1, src);
  } else {
    src.a = a.hq + (size_t)t32 * a.kbmax * 1024;
    src.as = a.hs + (size_t)t32 * a.kbmax * 32;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char*)&lds[0][0];
  const uint32_t lds1 = (uint32_t)(uintptr_t)(lds_char*)&lds[1][0];

  // Prologue: k-steps 0 and 1 in flight; wait for k-step 0.
  issue_weights<GATEUP>(src, 0, lds0, wave);
  issue_acts<GATEUP>(src, 0, lds0, wave, lane);
  // Down: the (token, slot) of this lane's CSR row wrow0 + lane%32, loaded
  // now (and first used in the epilogue) so that the load's latency hides
  // under the k loop.  Every wavefront issues both loads (the row clamped
  // into the CSR arrays), so that the vmcnt count below holds for all.
  int tok = -1, slt = -1;
  if (!GATEUP) {
    const int p_lane = min(wrow0 + (lane & 31), a.p_total - 1);
    tok = a.tok_i[p_lane];
    slt = a.tok_k[p_lane];
  }
  if (KS > 1) {
    issue_weights<GATEUP>(src, 1, lds1, wave);
    issue_acts<GATEUP>(src, 1, lds1, wave, lane);
    wait_copies_barrier_n<L::DMA + 2 * !GATEUP>();
  } else {
    wait_copies_barrier_0();
  }
  v16f acc[4];
  if (active) {
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = (v16f){0};
    Ops X, Y;
    ScalesT<GATEUP> s0, s1;
    Ctx cx;
    read_block<GATEUP>(lds[0], si, wave, lane, X);  // the wavefront's first block
    read_scales(lds[0], wave, lane, s0);
    v16i c;
    v16f cf, s;
    pipeline_init<GATEUP>(X, s0, si, lane, cx, c, cf, s);
    // Unrolled by two so that each buffer and scale set has a fixed role.
    if constexpr (S == 1) {
      for (int j = 0; j < KS; j += 2) {
        kstep<GATEUP>(src, j, KS, wave, lane, lds[0], lds[1], lds0, lds1, X, Y, s0, s1, cx, c, cf, s, acc);
        if (j + 1 < KS)
          kstep<GATEUP>(src, j + 1, KS, wave, lane, lds[1], lds[0], lds1, lds0, X, Y, s1, s0, cx, c, cf, s, acc);
      }
    } else {
      for (int j = 0; j < KS; j += 2) {
        kstep_split2<GATEUP>(src, j, KS, wave, lane, si, lds[0], lds[1], lds0, lds1, X, Y, s0, s1, cx, c, cf, s,
                             acc);
        if (j + 1 < KS)
          kstep_split2<GATEUP>(src, j + 1, KS, wave, lane, si, lds[1], lds[0], lds1, lds0, X, Y, s1, s0, cx, c,
                               cf, s, acc);
      }
    }
  } else if constexpr (S == 1) {
    // A wavefront past the tile's rows computes nothing but still does its
    // share of the copies and meets every barrier.
    for (int j = 0; j + 1 < KS; ++j) {
      if (j >= 1) issue_acts<GATEUP>(src, j + 1, (j & 1) ? lds0 : lds1, wave, lane);
      wait_copies_barrier_0();
      if (j + 2 < KS) issue_weights<GATEUP>(src, j + 2, (j & 1) ? lds1 : lds0, wave);
    }
  }
  // Every wavefront is out of the k loop, so LDS is free for the epilogue
  // (both epilogues transpose through it).  Split-K: the row group's partial
  // sums meet in its first wavefront, which alone runs the epilogue.
  if constexpr (S > 1)
    split_reduce(&lds[0][0], S, rg, si, lane, acc);
  else
    __syncthreads();
  if (!active || si != 0) return;
  epilogue<GATEUP, true>(a, &lds[0][0], lane, wave, t32, cs, g, wrow0, row_end, tok, slt, acc);
}

// The work of a (tile, strip) workgroup whose tile has one 32-row group: the
// three-stage pipeline of kstep1, then the fixed-order sum of the four
// wavefronts' partial accumulators and the epilogue in wavefront 0.
template <bool GATEUP>
__device__ __forceinline__ void tile_work1(const GemmArgs& a, char* lds, int lane, int wave, int T, int cs, int g,
                                           int row0, int row_end, int KS, const uint8_t* strip) {
  using L1 = Lay1<GATEUP>;
  const int si = wave;
  const int t32 = T * NWAVE;
  Src src;
  src.w = strip;
  src.o_w = lane * 16;
  src.o_ws = 16 * 1024 + wave * (GATEUP ? 256 : 512) + lane * 4;
  if constexpr (GATEUP) {
    src.a = a.gq;
    src.as = a.gqs + (size_t)t32 * (a.d_pad / QB) * 32;
    int t[MT_WAVE];
    load_row_tokens(a, T, 0, t);
    gather_offsets(a, t, 0, row0, row_end, lane, wave, src);
  } else {
    src.a = a.hq + (size_t)t32 * a.kbmax * 1024;
    src.as = a.hs + (size_t)t32 * a.kbmax * 32;
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_char*)lds;

  // Down: the (token, slot) of this lane's CSR row, loaded before any copy
  // (vector loads complete in order, so the waits below cover them too).
  int tok = -1, slt = -1;
  if (!GATEUP) {
    const int p_lane = min(row0 + (lane & 31), a.p_total - 1);
    tok = a.tok_i[p_lane];
    slt = a.tok_k[p_lane];
  }
  // Prologue: k-steps 0, 1 and 2 in flight; wait for k-step 0.
  issue_kstep1<GATEUP>(src, 0, lds_base, wave, lane);
  if (KS > 1) issue_kstep1<GATEUP>(src, 1, lds_base + L1::STAGE, wave, lane);
  if (KS > 2) issue_kstep1<GATEUP>(src, 2, lds_base + 2 * L1::STAGE, wave, lane);
  if (KS > 2)
    wait_copies_reads_barrier<2 * L1::DMA>();
  else if (KS > 1)
    wait_copies_reads_barrier<L1::DMA>();
  else
    wait_copies_reads_barrier<0>();

  v16f acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = (v16f){0};
  Ops X, Y;
  ScalesT<GATEUP> s0, s1;
  Ctx cx;
  read_block_at(lds, L1::A_OFF, si, lane, X);
  read_scales_at(lds, L1::AS_OFF, lane, s0);
  v16i c;
  v16f cf, s;
  pipeline_init<GATEUP>(X, s0, si, lane, cx, c, cf, s);
  // Unrolled by two so that each operand and scale set has a fixed role.
  for (int j = 0; j < KS; j += 2) {
    kstep1<GATEUP>(src, j, KS, wave, lane, si, lds, lds_base, X, Y, s0, s1, cx, c, cf, s, acc);
    if (j + 1 < KS) kstep1<GATEUP>(src, j + 1, KS, wave, lane, si, lds, lds_base, Y, X, s1, s0, cx, c, cf, s, acc);
  }
  split_reduce(lds, 4, 0, si, lane, acc);
  if (si != 0) return;
  epilogue<GATEUP, true>(a, lds, lane, 0, t32, cs, g, row0, row_end, tok, slt, acc);
}

template <bool GATEUP>
__global__ __launch_bounds__(256, 2) void grouped_gemm_kernel(GemmArgs a) {
  using L = Lay<GATEUP>;
  __shared__ __attribute__((aligned(1024))) char lds[2][L::STAGE];
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
  const int Tl = blk / nstrips, cs = blk - Tl * nstrips;
  // reverse: the same work in the opposite tile order, so that each XCD
  // starts on the tiles another finished last (serpentine chunk order)
  const int T = a.reverse ? n_tiles - 1 - Tl : Tl;
  const int32_t* ent = a.tiles + 4 + 3 * T;
  const int g = ent[0], row0 = ent[1], row_end = ent[2];
  // Gate/up: the tile's row tokens are brought into the scalar cache with
  // the table entry (their addresses need only T; each wavefront touches the
  // two 64-byte lines of a quarter of the tile), so that the entry and the
  // tokens cost one memory latency and the loads of the tile body hit.
  if constexpr (GATEUP) touch_row_tokens(a, T, wave);
  // (one test of all three fields, so that their loads go out together)
  if ((g < 0) | (g >= a.G) | (row0 < 0) | (row_end <= row0) | (row_end > a.p_total)) return;
  const bool shared = g >= a.E;
  const int Fg_pad = shared ? a.Fs_pad : a.F_pad;
  if (GATEUP && cs >= Fg_pad / GU_COLS) return;
  const int KB = GATEUP ? a.d_pad / QB : Fg_pad / QB;
  const int KS = KB / KSTEP;
  const uint8_t* strip = GATEUP ? (shared ? a.sh_gu : a.gu + (size_t)g * a.gu_group)
                                : (shared ? a.sh_dn : a.dn + (size_t)g * a.dn_group);
  strip += (size_t)cs * KS * L::W_BYTES;

  // Split-K: when the tile's rows fill only one (or two) of the four 32-row
  // wavefront slots, the wavefronts of each row group share its blocks (see
  // kstep1 and kstep_split2).
  const int nact = (min(row_end - row0, MT_WG) + MT_WAVE - 1) / MT_WAVE;
  if (nact >= 3)
    tile_work<GATEUP, 1>(a, lds, lane, wave, T, cs, g, row0, row_end, KS, strip);
  else if (nact == 2)
    tile_work<GATEUP, 2>(a, lds, lane, wave, T, cs, g, row0, row_end, KS, strip);
  else
    tile_work1<GATEUP>(a, &lds[0][0], lane, wave, T, cs, g, row0, row_end, KS, strip);
}

// The integer core of a grouped GEMM, exposed for parity checks: k-block kb
// of tile T against strip cs, through the product kernels' own path -- the
// same global->LDS copies of the same planes, the same LDS layout and operand
// reads, and the same int8 MFMA from the same accumulator bias -- with the
// bias subtracted again, so sums[r][c] is the exact int32 block sum of tile
// row r (wavefront r/32) and strip column c = 32 * tile + column.  acodes[r]
// receives the 32 activation codes the A operand held for row r; info =
// {group, first CSR row, end CSR row, tile count} (group -1: T is past the
// tile count; -2: a malformed tile entry; -3: strip or k-block outside the
// group's planes).  One workgroup, launched after a prefill call on the same
// workspace.
template <bool GATEUP>
__global__ __launch_bounds__(256) void block_sums_kernel(GemmArgs a, int T, int cs, int kb,
                                                         int32_t* __restrict__ sums,
                                                         int8_t* __restrict__ acodes,
                                                         int32_t* __restrict__ info) {
  using L = Lay<GATEUP>;
  __shared__ __attribute__((aligned(1024))) char lds[L::STAGE];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_tiles = min(a.tiles[0], a.tile_bound);
  auto fail = [&](int code, int g, int r0, int r1) {
    if (threadIdx.x == 0) {
      info[0] = code < 0 ? code : g;
      info[1] = r0;
      info[2] = r1;
      info[3] = n_tiles;
    }
  };
  if (T >= n_tiles) return fail(-1, 0, 0, 0);
  const int32_t* ent = a.tiles + 4 + 3 * T;
  const int g = ent[0], row0 = ent[1], row_end = ent[2];
  if (g < 0 || g >= a.G || row0 < 0 || row_end <= row0 || row_end > a.p_total) return fail(-2, 0, 0, 0);
  const bool shared = g >= a.E;
  const int Fg_pad = shared ? a.Fs_pad : a.F_pad;
  const int nstrips = GATEUP ? Fg_pad / GU_COLS : a.d_pad / DN_COLS;
  const int KB = GATEUP ? a.d_pad / QB : Fg_pad / QB;
  if (cs < 0 || cs >= nstrips || kb < 0 || kb >= KB) return fail(-3, 0, 0, 0);
  const int KS = KB / KSTEP;
  const uint8_t* strip = GATEUP ? (shared ? a.sh_gu : a.gu + (size_t)g * a.gu_group)
                                : (shared ? a.sh_dn : a.dn + (size_t)g * a.dn_group);
  strip += (size_t)cs * KS * L::W_BYTES;
  const int t32 = T * NWAVE + wave;
  Src src;
  src.w = strip;
  src.o_w = lane * 16;
  src.o_ws = 16 * 1024 + wave * (GATEUP ? 256 : 512) + lane * 4;
  if constexpr (GATEUP) {
    src.a = a.gq;
    src.as = a.gqs + (size_t)t32 * (a.d_pad / QB) * 32;
    int t[MT_WAVE];
    load_row_tokens(a, T, MT_WAVE * wave, t);
    gather_offsets(a, t, MT_WAVE * wave, row0, row_end, lane, -1, src);
  } else {
    src.a = a.hq + (size_t)t32 * a.kbmax * 1024;
    src.as = a.hs + (size_t)t32 * a.kbmax * 32;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char*)&lds[0];
  const int j = kb / KSTEP, b = kb % KSTEP;
  issue_weights<GATEUP>(src, j, lds0, wave);
  issue_acts<GATEUP>(src, j, lds0, wave, lane);
  wait_copies_barrier_0();
  Ops X;
  read_block<GATEUP>(lds, b, wave, lane, X);
  const int bias = GATEUP ? 0x4b400000 : 0x3fc00000;  // 1.5 * 2^23, 1.5f
  v16i magic;
#pragma unroll
  for (int v = 0; v < 16; ++v) magic[v] = bias;
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const v16i c = __builtin_amdgcn_mfma_i32_32x32x32_i8(X.a, X.b[tt], magic, 0, 0, 0);
#pragma unroll
    for (int v = 0; v < 16; ++v)
      sums[(size_t)(wave * 32 + out_row(v, lane)) * 128 + tt * 32 + (lane & 31)] = c[v] - bias;
  }
  *reinterpret_cast<v4i*>(acodes + (size_t)(wave * 32 + (lane & 31)) * 32 + 16 * (lane >> 5)) = X.a;
  fail(0, g, row0, row_end);
}

}  // namespace

hipError_t launch_block_sums(const GemmArgs& a, bool gateup, int tile, int strip, int kblock, int32_t* sums,
                             int8_t* acodes, int32_t* info, hipStream_t s) {
  if (gateup)
    block_sums_kernel<true><<<1, 256, 0, s>>>(a, tile, strip, kblock, sums, acodes, info);
  else
    block_sums_kernel<false><<<1, 256, 0, s>>>(a, tile, strip, kblock, sums, acodes, info);
  return hipGetLastError();
}

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
