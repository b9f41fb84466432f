// gemm_q4k.hip -- the grouped gate/up and down GEMMs on Q4_K expert weights.
//
// SharpInference #406 "References" names Q4_K next to Q8_0 as a weight
// format of the int8 MMQ path: int8 activation blocks of 32 against 4-bit
// weight codes.  A Q4_K super-block of 256 weights holds a binary16 scale d,
// a binary16 min dmin, eight 6-bit sub-block scales sc_j and mins m_j, and
// 4-bit codes q; weight i of sub-block j is d * sc_j * q_i - dmin * m_j.  A
// sub-block is 32 weights, so it lines up with one activation block.
//
// Arithmetic per 32-block b of weight row n against activation row m (codes
// a_i, scale sa_b), with D_b = d * sc_b and M_b = dmin * m_b:
//   sum_i sa_b a_i (D_b q_i - M_b) = sa_b D_b C_b - sa_b A_b M_b,
// C_b = sum_i a_i q_i (exact int32, the int8 MFMA on the codes widened to
// bytes) and A_b = sum_i a_i (exact integer).  D_b and M_b have up to 17
// significant bits, more than a binary16 holds, so the load-time repack
// stores each as a pair of binary16 values whose sum is the exact value (hi =
// the value rounded to binary16, lo = the remainder rounded to binary16; the
// remainder is exact unless it falls below the binary16 normal range, where
// its absolute error stays below 2^-25).
//   main term: the Q8_0 gate/up pipeline -- int8 MFMA from the 1.5 * 2^23
//     bias, the conversion MFMA (exactly float(C)), the scale MFMA with sa in
//     the K slot of block b and {D_hi, D_lo} in the two lane halves' slot b, so
//     S = sa * D_hi + sa * D_lo = sa * D rounded once, and the VALU fma
//     acc += float(C) * S;
//   min term: once per k-step and tile, v_mfma_f32_32x32x16_f16 adds
//     -sum_b P_b M_b into acc, P_b = sa_b A_b (exact in fp32) split into
//     {P_hi, P_lo} the same way, four exact products per block
//     (P_hi M_hi, P_hi M_lo, P_lo M_hi, P_lo M_lo) in 16 K slots.
//   A_b comes from the A operand registers: each lane sums its 16 codes with
//   v_dot4 against ones, and the two lanes of a row trade halves with one
//   v_permlane32_swap per k-step.
// Down uses the same pipeline (its fp32 output is final; the exact form
// costs it one more MFMA per block-tile than the Q8_0 down pipeline).
//
// Weight planes (per expert, written once by the repack): [strip][k-step]
// [12 KiB], strips and tiles as in the Q8_0 planes (gate/up: tiles 0,1 gate
// rows, tiles 2,3 the up rows of the same 64 columns; down: 4 tiles of the
// strip's 128 output rows).  A k-step (128 K values = 4 blocks) is
//   [0, 8 KiB)    codes, chunk (block i, tile t) of 512 B at (4 i + t) * 512:
//                 lane l (column l%32, half l/32) holds 8 bytes, dword 0 =
//                 codes 16h..16h+3 in the low nibbles and 16h+4..16h+7 in the
//                 high nibbles, dword 1 likewise for 16h+8..16h+15;
//   [8, 10 KiB)   D pairs, tile t at t * 512: lane l holds binary16 D_hi (half 0)
//                 or D_lo (half 1) of blocks 0..3 of its column;
//   [10, 12 KiB)  M pairs, tile t at t * 512: lane l holds {M_hi, M_lo} of
//                 blocks 2h and 2h+1 of its column.
// The activation side (slabs, scales, copies, barriers, operand reads one
// block ahead, the pinned two-tile-ahead MFMA pipeline and both epilogues) is
// that of the Q8_0 kernels.
#include "device_util.h"
#include "gemm_common.h"
#include "internal.h"

namespace moe {
namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int Q4_D_OFF = 8 * 1024;   // D pairs [tile] x 512 B
constexpr int Q4_M_OFF = 10 * 1024;  // M pairs [tile] x 512 B
static_assert(Q4_M_OFF + 4 * 512 == Q4K_KSTEP_BYTES, "Q4_K k-step layout");

// Stage layout of one k-step buffer: the weight k-step, then the activation
// chunks [wave][block] x 1 KiB and their scales [wave][32 rows][4 blocks].
struct LayQ4 {
  static constexpr int A_OFF = Q4K_KSTEP_BYTES;
  static constexpr int AS_OFF = A_OFF + NWAVE * KSTEP * 1024;
  static constexpr int STAGE = AS_OFF + NWAVE * 32 * KSTEP * 2;  // 29 KiB
  static constexpr int DMA = Q4K_KSTEP_BYTES / 1024 / NWAVE + KSTEP + 1;  // copies per wavefront per k-step
};
static_assert(NWAVE * 32 * EPI_STRIDE * 4 <= 2 * LayQ4::STAGE, "epilogue scratch must fit in the buffers");
static_assert(2 * 2 * LayQ4::STAGE <= 160 * 1024, "two workgroups per CU must fit in the LDS");
static_assert(LayQ4::STAGE % 1024 == 0, "stage alignment");

// This wavefront's copies of k-step j into the buffer at LDS address L: 1 KiB
// pieces wave, wave + 4 and wave + 8 of the weight k-step (whose LDS image is
// its HBM image), and its 4 activation chunks and their scales.  The part
// forms issue one piece per tile of a block (the hook of compute_block), so
// that a wavefront's copies go out between matrix instructions.
__device__ __forceinline__ void issue_weights_q4(const Src& s, int j, uint32_t L, int wave) {
  const uint8_t* w = s.w + (size_t)j * Q4K_KSTEP_BYTES;
#pragma unroll
  for (int i = 0; i < 3; ++i) dma16(w + (wave + 4 * i) * 1024, s.o_w, L + (wave + 4 * i) * 1024);
}
__device__ __forceinline__ void issue_weights_part_q4(const Src& s, int j, uint32_t L, int wave, int p) {
  const uint8_t* w = s.w + (size_t)j * Q4K_KSTEP_BYTES;
  if (p < 3) dma16(w + (wave + 4 * p) * 1024, s.o_w, L + (wave + 4 * p) * 1024);
}
template <bool GATEUP>
__device__ __forceinline__ void issue_acts_q4(const Src& s, int j, uint32_t L, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < KSTEP; ++i)
    dma_act_chunk<GATEUP>(s, j, i, lane, L + LayQ4::A_OFF + (wave * KSTEP + i) * 1024);
  dma_act_scales<GATEUP>(s, j, lane, L + LayQ4::AS_OFF + wave * 256);
}
template <bool GATEUP>
__device__ __forceinline__ void issue_acts_part_q4(const Src& s, int j, uint32_t L, int wave, int lane, int p) {
  if (p < 2) {
#pragma unroll
    for (int i = 2 * p; i < 2 * p + 2; ++i)
      dma_act_chunk<GATEUP>(s, j, i, lane, L + LayQ4::A_OFF + (wave * KSTEP + i) * 1024);
  } else if (p == 2) {
    dma_act_scales<GATEUP>(s, j, lane, L + LayQ4::AS_OFF + wave * 256);
  }
}

// Register operands of one block: this wavefront's A chunk and the packed
// codes of the 4 B chunks.
struct OpsQ4 {
  v4i a;
  uint2 b[4];
};

// a_off: LDS offset of the 32-row activation slab within the stage buffer.
__device__ __forceinline__ void read_block_q4_at(const char* buf, int a_off, int b, int lane, OpsQ4& o) {
  // A: row lane%32, piece 2b + lane/32 of the k-step at its swizzled place
  const int r = lane & 31, p = 2 * b + (lane >> 5);
  o.a = *reinterpret_cast<const v4i*>(buf + a_off + r * 128 + ((p ^ (r & 7)) << 4));
#pragma unroll
  for (int t = 0; t < 4; ++t) o.b[t] = *reinterpret_cast<const uint2*>(buf + (b * 4 + t) * 512 + lane * 8);
}
__device__ __forceinline__ void read_block_q4(const char* buf, int b, int wave, int lane, OpsQ4& o) {
  read_block_q4_at(buf, LayQ4::A_OFF + wave * (KSTEP * 1024), b, lane, o);
}

// The k-step's scale operands: per tile the D and M pairs of this lane's
// column, and the activation scales of this lane's row (blocks 0..3).
struct ScalesQ4 {
  uint2 dp[4];
  uint2 mp[4];
  uint2 sa;
};

// as_off: LDS offset of the slab's activation scales within the stage buffer;
// WITH_M: also the M pairs (the one-row-group form reads them separately).
template <bool WITH_M = true>
__device__ __forceinline__ void read_scales_q4_at(const char* buf, int as_off, int lane, ScalesQ4& s) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    s.dp[t] = *reinterpret_cast<const uint2*>(buf + Q4_D_OFF + t * 512 + lane * 8);
    if (WITH_M) s.mp[t] = *reinterpret_cast<const uint2*>(buf + Q4_M_OFF + t * 512 + lane * 8);
  }
  s.sa = *reinterpret_cast<const uint2*>(buf + as_off + (lane & 31) * 8);
}
__device__ __forceinline__ void read_scales_q4(const char* buf, int wave, int lane, ScalesQ4& s) {
  read_scales_q4_at(buf, LayQ4::AS_OFF + wave * 256, lane, s);
}

// The 16 codes of a packed B piece widened to bytes (0..15), in K order.
__device__ __forceinline__ v4i widen_codes(uint2 p) {
  const uint32_t m = 0x0f0f0f0fu;
  return (v4i){(int)(p.x & m), (int)((p.x >> 4) & m), (int)(p.y & m), (int)((p.y >> 4) & m)};
}

// A operand of the scale MFMA for block b: K slot b of both lane halves holds
// this row's activation scale (half 0 meets D_hi, half 1 D_lo).
__device__ __forceinline__ v4h sa_slot_q4(const uint2 sa, int b) {
  const uint32_t m = (b & 1) ? 0xffff0000u : 0x0000ffffu;
  return b < 2 ? as_v4h(sa.x & m, 0u) : as_v4h(0u, sa.y & m);
}

// Sum of this lane's 16 activation codes of a block, plus 2048 (so that the
// two halves of a row, packed 16 bits each, add without borrows).
__device__ __forceinline__ uint32_t half_code_sum(const v4i a) {
  int s = __builtin_amdgcn_sdot4(a.x, 0x01010101, 2048, false);
  s = __builtin_amdgcn_sdot4(a.y, 0x01010101, s, false);
  s = __builtin_amdgcn_sdot4(a.z, 0x01010101, s, false);
  return (uint32_t)__builtin_amdgcn_sdot4(a.w, 0x01010101, s, false);
}

// This lane's biased half code sums of a k-step's 4 blocks, 16 bits each:
// x = blocks 0 and 1, y = blocks 2 and 3 (low half first).
constexpr uint32_t PS_ZERO = 0x08000800u;  // both fields at the bias: P = 0

// A operand of the min-term MFMA of a k-step: lane half h covers blocks 2h
// and 2h+1 of its row, K slots {-P_hi, -P_hi, -P_lo, -P_lo} per block against
// the B slots {M_hi, M_lo, M_hi, M_lo}.  The partner lane (l ^ 32) supplies
// the other halves of the sums.
__device__ __forceinline__ v8h min_term_a(const uint2 ps, const uint2 sa, int lane) {
  const bool hi_half = lane >= 32;
  const uint32_t own = hi_half ? ps.y : ps.x;
  const uint32_t give = hi_half ? ps.x : ps.y;
  // The two results are this lane's own value and its partner's, in an order
  // that depends on the lane half; their sum minus the own value is the
  // partner's.
  const auto sw = __builtin_amdgcn_permlane32_swap(give, give, false, false);
  const uint32_t full = own + (sw[0] + sw[1] - give);  // fields: A_b + 4096
  const uint32_t s2 = hi_half ? sa.y : sa.x;
  uint32_t dw[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int A = (int)((full >> (16 * i)) & 0xffffu) - 4096;
    const float sa_f = (float)__builtin_bit_cast(_Float16, (uint16_t)(s2 >> (16 * i)));
    const float np = -((float)A * sa_f);  // exact: |A| < 2^12, sa has 11 significant bits
    const _Float16 h = (_Float16)np;
    const _Float16 l = (_Float16)(np - (float)h);
    const uint32_t hb = __builtin_bit_cast(uint16_t, h), lb = __builtin_bit_cast(uint16_t, l);
    dw[2 * i] = hb | (hb << 16);
    dw[2 * i + 1] = lb | (lb << 16);
  }
  return __builtin_bit_cast(v8h, make_uint4(dw[0], dw[1], dw[2], dw[3]));
}

__device__ __forceinline__ v8h min_term_b(const uint2 mp) {
  return __builtin_bit_cast(v8h, make_uint4(mp.x, mp.x, mp.y, mp.y));
}

// One block (4 tiles) of the pipeline, two tiles ahead as the Q8_0 gate/up
// pipeline: per tile t the int8 MFMA(t+2) on the widened codes, a third of
// acc(t) = fma(cf(t), s(t), acc(t)), the conversion MFMA(t+1), a third, the
// scale MFMA(t+1), the last third; in the k-step's last block (last) the
// min-term MFMA of tile t follows, with the k-step's M pairs mp.  ps collects
// the half code sums of the k-step's blocks.
template <typename H = NoHook>
__device__ __forceinline__ void compute_block_q4(const OpsQ4& o, const ScalesQ4& sc, int b, const OpsQ4& on,
                                                 const ScalesQ4& sn, int bn, bool last, const uint2 (&mp)[4],
                                                 const Ctx& cx, int lane, uint2& ps, v16i& dn, v16f& cf,
                                                 v16f& s, v16f (&acc)[4], const H& hook = H()) {
  const v16f zf = {0};
  // (b may be a run-time value in the split forms: selects, not an indexed store)
  const uint32_t hs = half_code_sum(o.a);
  const uint32_t field = (b & 1) ? (hs << 16) : hs, keep = (b & 1) ? 0x0000ffffu : 0xffff0000u;
  if (b < 2)
    ps.x = (ps.x & keep) | field;
  else
    ps.y = (ps.y & keep) | field;
  v8h pa;
  if (last) pa = min_term_a(ps, sc.sa, lane);
  v4h sav = sa_slot_q4(sc.sa, b);
  v4h savn = sa_slot_q4(sn.sa, bn);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    v16i dnn = t < 2 ? __builtin_amdgcn_mfma_i32_32x32x32_i8(o.a, widen_codes(o.b[t + 2]), cx.magic, 0, 0, 0)
                     : __builtin_amdgcn_mfma_i32_32x32x32_i8(on.a, widen_codes(on.b[t - 2]), cx.magic, 0, 0, 0);
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
    v16f sx = t < 3 ? __builtin_amdgcn_mfma_f32_32x32x8f16(sav, as_v4h(sc.dp[t + 1]), zf, 0, 0, 0)
                    : __builtin_amdgcn_mfma_f32_32x32x8f16(savn, as_v4h(sn.dp[0]), zf, 0, 0, 0);
    anchor(sx, acc[t]);
#pragma unroll
    for (int v = 10; v < 16; ++v) acc[t][v] = __builtin_fmaf(cf[v], s[v], acc[t][v]);
    anchor(acc[t]);
    if (last) {
      // the B operand built here, not hoisted: one at a time is live
      v8h mb = min_term_b(mp[t]);
      anchor(mb, acc[t]);
      acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa, mb, acc[t], 0, 0, 0);
      anchor(acc[t]);
    }
    dn = dnn;
    cf = cfn;
    s = sx;
  }
}

// K-step j of an active wavefront, from buffer `cur`; k-step j+1 is (or, for
// the last k-step, stale data standing in for it is) in `nxt`.  Copies,
// barrier and operand reads are placed as in the Q8_0 k-step: the
// activation half of k-step j+1 goes out during block 0, the barrier comes
// before block 3, and the weights of k-step j+2 go out during block 3.
template <bool GATEUP>
__device__ __forceinline__ void kstep_q4(const Src& src, int j, int KS, int wave, int lane, const char* cur,
                                         const char* nxt, uint32_t cur_lds, uint32_t nxt_lds, OpsQ4& X, OpsQ4& Y,
                                         const ScalesQ4& sc, ScalesQ4& sn, const Ctx& cx, uint2& ps,
                                         v16i& c, v16f& cf, v16f& s, v16f (&acc)[4]) {
  const bool acts = j >= 1 && j + 1 < KS;
  read_block_q4(cur, 1, wave, lane, Y);
  compute_block_q4(X, sc, 0, Y, sc, 1, false, sc.mp, cx, lane, ps, c, cf, s, acc, [&](int t) {
    if (acts) issue_acts_part_q4<GATEUP>(src, j + 1, nxt_lds, wave, lane, t);
  });
  read_block_q4(cur, 2, wave, lane, X);
  compute_block_q4(Y, sc, 1, X, sc, 2, false, sc.mp, cx, lane, ps, c, cf, s, acc);
  read_block_q4(cur, 3, wave, lane, Y);
  compute_block_q4(X, sc, 2, Y, sc, 3, false, sc.mp, cx, lane, ps, c, cf, s, acc);
  if (j + 1 < KS) wait_copies_barrier_0();
  const bool weights = j + 2 < KS;
  read_block_q4(nxt, 0, wave, lane, X);
  read_scales_q4(nxt, wave, lane, sn);
  compute_block_q4(Y, sc, 3, X, sn, 0, true, sc.mp, cx, lane, ps, c, cf, s, acc, [&](int t) {
    if (weights) issue_weights_part_q4(src, j + 2, cur_lds, wave, t);
  });
}

// Split-K k-step of a two-row-group tile (the split-K follow-up of #406
// "References"): the two wavefronts of a row group compute blocks si and
// si + 2 of every k-step into their own accumulators (the min term over those
// two blocks only: the code sums of the other two stay at their bias, so
// their P is zero).  Copies, barrier and their placement are those of
// kstep_q4; each wavefront copies its row group's slab into its own area.
template <bool GATEUP>
__device__ __forceinline__ void kstep_q4_split2(const Src& src, int j, int KS, int wave, int lane, int si,
                                                const char* cur, const char* nxt, uint32_t cur_lds,
                                                uint32_t nxt_lds, OpsQ4& X, OpsQ4& Y, const ScalesQ4& sc,
                                                ScalesQ4& sn, const Ctx& cx, uint2& ps, v16i& c, v16f& cf,
                                                v16f& s, v16f (&acc)[4]) {
  const bool acts = j >= 1 && j + 1 < KS;
  read_block_q4(cur, si + 2, wave, lane, Y);
  compute_block_q4(X, sc, si, Y, sc, si + 2, false, sc.mp, cx, lane, ps, c, cf, s, acc, [&](int t) {
    if (acts) issue_acts_part_q4<GATEUP>(src, j + 1, nxt_lds, wave, lane, t);
  });
  if (j + 1 < KS) wait_copies_barrier_0();
  const bool weights = j + 2 < KS;
  read_block_q4(nxt, si, wave, lane, X);
  read_scales_q4(nxt, wave, lane, sn);
  compute_block_q4(Y, sc, si + 2, X, sn, si, true, sc.mp, cx, lane, ps, c, cf, s, acc, [&](int t) {
    if (weights) issue_weights_part_q4(src, j + 2, cur_lds, wave, t);
  });
}

// One-row-group tiles: the four wavefronts split every k-step (wavefront si
// computes block si), so the k loop is bound by the copies' latency; as in
// the Q8_0 kernel these tiles keep three k-steps in LDS (a stage holds the
// weight k-step and the single activation slab) and issue k-step j+3's copies
// at k-step j's barrier.
struct Lay1Q4 {
  static constexpr int A_OFF = Q4K_KSTEP_BYTES;                    // the slab [row][128 B]
  static constexpr int AS_OFF = A_OFF + KSTEP * 1024;              // its scales [32 rows][4 blocks]
  static constexpr int STAGE = AS_OFF + 32 * KSTEP * 2;            // 16.25 KiB
  static constexpr int DMA = Q4K_KSTEP_BYTES / 1024 / NWAVE + 2;   // copies per wavefront per k-step
};
static_assert(3 * Lay1Q4::STAGE <= 2 * LayQ4::STAGE, "three stages must fit in the LDS buffers");
// Down: the (token, slot) of each lane's CSR row, copied into LDS past the
// three stages (and past the split reduction's buffers), so that they occupy
// no registers during the k loop.
constexpr int T1_PAIR_OFF = 3 * Lay1Q4::STAGE;
static_assert(T1_PAIR_OFF + 2 * 64 * 4 <= 2 * LayQ4::STAGE, "pair slots must fit in the LDS buffers");
static_assert(3 * 64 * 64 * 4 <= T1_PAIR_OFF, "the split reduction must not reach the pair slots");
// Gate/up: each wavefront's gather offset (o_a[0] per lane) in the same place
// (down's pair slots), read back before each k-step's copies.
constexpr int T1_GATHER_OFF = T1_PAIR_OFF;
static_assert(T1_GATHER_OFF + NWAVE * 64 * 4 <= 2 * LayQ4::STAGE, "gather offsets must fit in the LDS buffers");
static_assert(Lay1Q4::STAGE % 256 == 0, "stage alignment");

// This wavefront's copies of k-step j into the stage at LDS address L: its
// three weight pieces, chunk `wave` of the slab and the slab's scales (every
// wavefront copies the same 256 bytes, so that all issue the same number).
template <bool GATEUP>
__device__ __forceinline__ void issue_kstep1_q4(const Src& s, int j, uint32_t L, int wave, int lane) {
  issue_weights_q4(s, j, L, wave);
  dma_act_chunk<GATEUP>(s, j, GATEUP ? 0 : wave, lane, L + Lay1Q4::A_OFF + wave * 1024);
  dma_act_scales<GATEUP>(s, j, lane, L + Lay1Q4::AS_OFF);
}

// K-step j of a one-row-group tile.  On entry X and sc hold block si of
// k-step j; k-steps j+1 and j+2 are in flight.  The barrier publishes k-step
// j+1 and proves that every wavefront has read k-step j, whose stage then
// receives k-step j+3.  On exit Y and sn hold block si of k-step j+1.
template <bool GATEUP>
__device__ __forceinline__ void kstep1_q4(const Src& src, int j, int KS, int wave, int lane, int si, const char* lds,
                                          uint32_t lds_base, const OpsQ4& X, OpsQ4& Y, const ScalesQ4& sc,
                                          ScalesQ4& sn, const Ctx& cx, uint2& ps, v16i& c, v16f& cf, v16f& s,
                                          v16f (&acc)[4]) {
  const int st = j % 3;
  const int sn1 = st == 2 ? 0 : st + 1;
  // This k-step's M pairs, read here rather than with its other scales one
  // k-step earlier (fewer registers live across a k-step); its stage takes
  // new copies only after the barrier below, which waits for these reads.
  uint2 mp[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) mp[t] = *reinterpret_cast<const uint2*>(lds + st * Lay1Q4::STAGE + Q4_M_OFF + t * 512 + lane * 8);
  if (j + 1 < KS) {
    if (j + 2 < KS)
      wait_copies_reads_barrier<Lay1Q4::DMA>();
    else
      wait_copies_reads_barrier<0>();
    if (j + 3 < KS) {
      if constexpr (GATEUP) {
        // the gather offset waits in LDS between k-steps (no register held)
        Src s2 = src;
        s2.o_a[0] = *reinterpret_cast<const uint32_t*>(lds + T1_GATHER_OFF + wave * 256 + lane * 4);
        issue_kstep1_q4<true>(s2, j + 3, lds_base + st * Lay1Q4::STAGE, wave, lane);
      } else {
        issue_kstep1_q4<false>(src, j + 3, lds_base + st * Lay1Q4::STAGE, wave, lane);
      }
    }
  }
  const char* nb = lds + sn1 * Lay1Q4::STAGE;
  read_block_q4_at(nb, Lay1Q4::A_OFF, si, lane, Y);
  read_scales_q4_at<false>(nb, Lay1Q4::AS_OFF, lane, sn);
  compute_block_q4(X, sc, si, Y, sn, si, true, mp, cx, lane, ps, c, cf, s, acc);
}

// Pipeline constants and the state of (block si, tile 0) from the first
// block's operands X and scales s0: the int8 MFMA of tile 1, float(C) and the
// scale product of tile 0.
__device__ __forceinline__ void pipeline_init_q4(const OpsQ4& X, const ScalesQ4& s0, int si, int lane, Ctx& cx,
                                                 v16i& c, v16f& cf, v16f& s) {
  const v16f zf = {0};
#pragma unroll
  for (int v = 0; v < 16; ++v) cx.magic[v] = 0x4b400000;  // 1.5 * 2^23
  anchor(cx.magic);
  const _Float16 h0 = 0;
  cx.sub_a = lane < 32 ? (v4h){(_Float16)-3072.0f, h0, h0, h0} : (v4h){h0, h0, h0, h0};
  cx.sub_b = lane < 32 ? (v4h){(_Float16)4096.0f, h0, h0, h0} : (v4h){h0, h0, h0, h0};
  anchor(cx.sub_a, cx.sub_b);
  const v16i d0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(X.a, widen_codes(X.b[0]), cx.magic, 0, 0, 0);
  c = __builtin_amdgcn_mfma_i32_32x32x32_i8(X.a, widen_codes(X.b[1]), cx.magic, 0, 0, 0);
  cf = __builtin_amdgcn_mfma_f32_32x32x8f16(cx.sub_a, cx.sub_b, __builtin_bit_cast(v16f, d0), 0, 0, 0);
  s = __builtin_amdgcn_mfma_f32_32x32x8f16(sa_slot_q4(s0.sa, si), as_v4h(s0.dp[0]), zf, 0, 0, 0);
}

// One (tile, strip) workgroup whose tile has three or four 32-row groups (S =
// 1: wavefront w computes row group w; a wavefront past the tile's rows only
// copies and meets the barriers) or two (S = 2: kstep_q4_split2, the row
// group's partial sums added in a fixed order), then the format-independent
// epilogue.  Each S is a self-contained body with its own register allocation.
template <bool GATEUP, int S>
__device__ __forceinline__ void tile_work_q4(const GemmArgs& a, char (&lds)[2][LayQ4::STAGE], int lane, int wave,
                                             int T, int cs, int g, int row0, int row_end, int KS,
                                             const uint8_t* strip) {
  static_assert(S == 1 || S == 2, "split factors of tile_work_q4");
  const int rg = wave / S, si = wave - rg * S;
  const int wrow0 = row0 + MT_WAVE * rg;
  const bool active = wrow0 < row_end;  // every wavefront when S > 1
  const int t32 = T * NWAVE + rg;
  Src src;
  src.w = strip;
  src.o_w = lane * 16;
  src.o_ws = 0;
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

  // Prologue: k-steps 0 and 1 in flight, the down rows' (token, slot) loads
  // between them (issued by every wavefront, so that the vmcnt count holds
  // for all); wait for k-step 0.
  issue_weights_q4(src, 0, lds0, wave);
  issue_acts_q4<GATEUP>(src, 0, lds0, wave, lane);
  int tok = -1, slt = -1;
  if (!GATEUP) {
    const int p_lane = min(wrow0 + (lane & 31), a.p_total - 1);
    tok = a.tok_i[p_lane];
    slt = a.tok_k[p_lane];
  }
  if (KS > 1) {
    issue_weights_q4(src, 1, lds1, wave);
    issue_acts_q4<GATEUP>(src, 1, lds1, wave, lane);
    wait_copies_barrier_n<LayQ4::DMA + 2 * !GATEUP>();
  } else {
    wait_copies_barrier_0();
  }
  v16f acc[4];
  if (active) {
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = (v16f){0};
    OpsQ4 X, Y;
    ScalesQ4 s0, s1;
    Ctx cx;
    read_block_q4(lds[0], si, wave, lane, X);
    read_scales_q4(lds[0], wave, lane, s0);
    v16i c;
    v16f cf, s;
    pipeline_init_q4(X, s0, si, lane, cx, c, cf, s);
    uint2 ps = make_uint2(PS_ZERO, PS_ZERO);  // code sums of blocks this wavefront skips stay zero
    // Unrolled by two so that each buffer and scale set has a fixed role.
    for (int j = 0; j < KS; j += 2) {
      if constexpr (S == 1) {
        kstep_q4<GATEUP>(src, j, KS, wave, lane, lds[0], lds[1], lds0, lds1, X, Y, s0, s1, cx, ps, c, cf, s, acc);
        if (j + 1 < KS)
          kstep_q4<GATEUP>(src, j + 1, KS, wave, lane, lds[1], lds[0], lds1, lds0, X, Y, s1, s0, cx, ps, c, cf, s, acc);
      } else {
        kstep_q4_split2<GATEUP>(src, j, KS, wave, lane, si, lds[0], lds[1], lds0, lds1, X, Y, s0, s1, cx, ps, c, cf, s,
                        acc);
        if (j + 1 < KS)
          kstep_q4_split2<GATEUP>(src, j + 1, KS, wave, lane, si, lds[1], lds[0], lds1, lds0, X, Y, s1, s0, cx, ps, c, cf,
                          s, acc);
      }
    }
  } else if constexpr (S == 1) {
    for (int j = 0; j + 1 < KS; ++j) {
      if (j >= 1) issue_acts_q4<GATEUP>(src, j + 1, (j & 1) ? lds0 : lds1, wave, lane);
      wait_copies_barrier_0();
      if (j + 2 < KS) issue_weights_q4(src, j + 2, (j & 1) ? lds1 : lds0, wave);
    }
  }
  // gate/up: every wavefront is out of the k loop, so LDS is free for the
  // epilogue's scratch.  Split-K: the row group's partial sums meet in its
  // first wavefront, which alone runs the epilogue.
  if constexpr (S > 1)
    split_reduce(&lds[0][0], S, rg, si, lane, acc);
  else if (GATEUP)
    __syncthreads();
  if (!active || si != 0) return;
  epilogue<GATEUP>(a, &lds[0][0], lane, wave, t32, cs, g, wrow0, row_end, tok, slt, acc);
}

// A (tile, strip) workgroup whose tile has one 32-row group: the three-stage
// pipeline of kstep1_q4, the fixed-order sum of the four wavefronts' partial
// accumulators, and the epilogue in wavefront 0.
template <bool GATEUP>
__device__ __forceinline__ void tile_work1_q4(const GemmArgs& a, char* lds, int lane, int wave, int T, int cs, int g,
                                              int row0, int row_end, int KS, const uint8_t* strip) {
  const int si = wave;
  const int t32 = T * NWAVE;
  Src src;
  src.w = strip;
  src.o_w = lane * 16;
  src.o_ws = 0;
  if constexpr (GATEUP) {
    src.a = a.gq;
    src.as = a.gqs + (size_t)t32 * (a.d_pad / QB) * 32;
    int t[MT_WAVE];
    load_row_tokens(a, T, 0, t);
    gather_offsets(a, t, 0, row0, row_end, lane, wave, src);
    *reinterpret_cast<uint32_t*>(lds + T1_GATHER_OFF + wave * 256 + lane * 4) = src.o_a[0];
  } else {
    src.a = a.hq + (size_t)t32 * a.kbmax * 1024;
    src.as = a.hs + (size_t)t32 * a.kbmax * 32;
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_char*)lds;

  // Down: the (token, slot) of this lane's CSR row, copied into LDS before
  // any other copy (vector loads complete in order, so the waits below cover
  // them too; every wavefront issues the same two copies).
  if (!GATEUP) {
    const int p_lane = min(row0 + (lane & 31), a.p_total - 1);
    dma4(a.tok_i, (uint32_t)p_lane * 4, lds_base + T1_PAIR_OFF);
    dma4(a.tok_k, (uint32_t)p_lane * 4, lds_base + T1_PAIR_OFF + 256);
  }
  // Prologue: k-steps 0, 1 and 2 in flight; wait for k-step 0.
  issue_kstep1_q4<GATEUP>(src, 0, lds_base, wave, lane);
  if (KS > 1) issue_kstep1_q4<GATEUP>(src, 1, lds_base + Lay1Q4::STAGE, wave, lane);
  if (KS > 2) issue_kstep1_q4<GATEUP>(src, 2, lds_base + 2 * Lay1Q4::STAGE, wave, lane);
  if (KS > 2)
    wait_copies_reads_barrier<2 * Lay1Q4::DMA>();
  else if (KS > 1)
    wait_copies_reads_barrier<Lay1Q4::DMA>();
  else
    wait_copies_reads_barrier<0>();

  v16f acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = (v16f){0};
  OpsQ4 X, Y;
  ScalesQ4 s0, s1;
  Ctx cx;
  read_block_q4_at(lds, Lay1Q4::A_OFF, si, lane, X);
  read_scales_q4_at<false>(lds, Lay1Q4::AS_OFF, lane, s0);
  v16i c;
  v16f cf, s;
  pipeline_init_q4(X, s0, si, lane, cx, c, cf, s);
  uint2 ps = make_uint2(PS_ZERO, PS_ZERO);
  for (int j = 0; j < KS; j += 2) {
    kstep1_q4<GATEUP>(src, j, KS, wave, lane, si, lds, lds_base, X, Y, s0, s1, cx, ps, c, cf, s, acc);
    if (j + 1 < KS) kstep1_q4<GATEUP>(src, j + 1, KS, wave, lane, si, lds, lds_base, Y, X, s1, s0, cx, ps, c, cf, s, acc);
  }
  split_reduce(lds, 4, 0, si, lane, acc);
  if (si != 0) return;
  if constexpr (GATEUP) {
    epilogue<true>(a, lds, lane, 0, t32, cs, g, row0, row_end, -1, -1, acc);
  } else {
    const int* pairs = reinterpret_cast<const int*>(lds + T1_PAIR_OFF);
    epilogue_down(a, lane, cs, g, partial_row(a, lane, row0, row_end, pairs[lane], pairs[64 + lane]), acc);
  }
}

// Grouped Q4_K GEMM over the tile table, with the workgroup numbering of the
// Q8_0 kernel (tile-major, strips inner, contiguous ranges per XCD).  The
// down epilogue's 2^e rescaling is a no-op here (the Q4_K weights' exponents
// are all zero).
template <bool GATEUP>
__global__ __launch_bounds__(256, 2) void grouped_gemm_q4k_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[2][LayQ4::STAGE];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_tiles = min(a.tiles[0], a.tile_bound);
  const int nstrips = GATEUP ? max(a.F_pad, a.Fs_pad) / GU_COLS : a.d_pad / DN_COLS;
  if (n_tiles <= 0) return;
  const int n_valid = n_tiles * nstrips;
  const int per_xcd = (n_valid + 7) >> 3;
  const int slot = (int)blockIdx.x >> 3;
  if (slot >= per_xcd) return;
  const int blk = ((int)blockIdx.x & 7) * per_xcd + slot;
  if (blk >= n_valid) return;
  const int Tl = blk / nstrips, cs = blk - Tl * nstrips;
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
  strip += (size_t)cs * KS * Q4K_KSTEP_BYTES;
  // Split-K when the tile's rows fill only one or two of the four 32-row
  // wavefront slots (the skew-aware tiles of the Q8_0 kernel).
  const int nact = (min(row_end - row0, MT_WG) + MT_WAVE - 1) / MT_WAVE;
  if (nact >= 3)
    tile_work_q4<GATEUP, 1>(a, lds, lane, wave, T, cs, g, row0, row_end, KS, strip);
  else if (nact == 2)
    tile_work_q4<GATEUP, 2>(a, lds, lane, wave, T, cs, g, row0, row_end, KS, strip);
  else
    tile_work1_q4<GATEUP>(a, &lds[0][0], lane, wave, T, cs, g, row0, row_end, KS, strip);
}

}  // namespace

hipError_t launch_gateup_q4k(const GemmArgs& a, hipStream_t s) {
  const long wgs = (long)a.tile_bound * (max(a.F_pad, a.Fs_pad) / GU_COLS);
  grouped_gemm_q4k_kernel<true><<<grid_for(wgs), 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_down_q4k(const GemmArgs& a, hipStream_t s) {
  const long wgs = (long)a.tile_bound * (a.d_pad / DN_COLS);
  grouped_gemm_q4k_kernel<false><<<grid_for(wgs), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
