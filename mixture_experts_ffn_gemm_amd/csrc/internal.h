// internal.h -- private declarations of libmoe_ffn (HIP, gfx950 only).
//
// Data layout in HBM (all planes are library-owned, built at load time):
//
//   router_wt   fp32 [d/4][E64][4]   the router matrix transposed so that lane e
//                                    of a wavefront reads expert e's 4 weights
//                                    for 4 consecutive j in one 16-byte load;
//                                    E64 = E rounded up to 64, zero rows past E.
//   gate/up     per expert [F_pad/64 strips][d_pad/128 k-steps][17 KiB]; a k-step
//               block is 16 chunks of 1 KiB [block i (4)][tile tt (4)] followed by
//               1 KiB of binary16 scales [tt][32 rows][4 blocks].  A chunk is one
//               32x32x32 MFMA B operand: [half of the 32-byte block][32 rows][16 B],
//               so lane l of a wavefront reads bytes [16 l, 16 l + 16).  Strip c
//               holds tiles tt = 0,1: gate rows 64c + 32tt + r; tt = 2,3: the up
//               rows 64c + 32(tt-2) + r (so gate and up of one column meet in one lane).
//   down        per expert [d_pad/128 strips][F_pad/128 k-steps][18 KiB], tile tt =
//               down rows 128c + 32tt + r.  The 16 code chunks are followed by
//               2 KiB of binary16 scale pairs [tt][half][32 rows][4]: half h of
//               row r holds {W, W/2} of blocks 2h and 2h+1, where W = scale *
//               2^(23 - e) and e = dn_exp[group] is the smallest exponent >= 0
//               that keeps every W of the group finite (so W and W/2 are exact).
//               Lane l of a wavefront reads bytes [8 l, 8 l + 8) of a tile's 512.
//   The shared expert has its own planes of the same form (F replaced by Fs).
//   Padding rows/blocks hold zero codes and zero scales.
//   Q4_K weights use the same strips and tiles with 12 KiB k-steps (4-bit
//   codes and binary16 {hi, lo} pairs of the sub-block scales and mins; the
//   layout is described in gemm_q4k.hip); their dn_exp entries are zero.
//   Q3_K weights are expanded at load into Q8_0 rows holding the same values
//   exactly (repack.hip) and then use the Q8_0 planes.
//
// Workspace (per call, caller-allocated, carved by ws_layout()):
//   logits fp32 [N][E]; ids, rank i32 [N][k]; w fp32 [N][k]; gs fp32 [N];
//   hist i32 [ceil(N/8)][E]; exp_start i32 [E+2]; tok_i, tok_k i32 [N*k + N];
//   row_tok i32 [T_bound][128]  (the token of row i of tile T at T*128 + i,
//                               the tile's rows being CSR rows row0 + i; rows
//                               past a group's end are not written);
//   tiles i32 [4 + 3*T_bound]  (tiles[0] = number of 128-row tiles, then
//                               {group, first CSR row, end CSR row} per tile);
//   gq int8 [N][d_pad]          (token-major activation codes, zero past d:
//                               the gate/up GEMM gathers its rows from here);
//   gxs fp16 [N][d_pad/32]      (their scales token-major, E > 64 only: the
//                               routing launch quantises there);
//   gqs fp16 [4*T_bound][d_pad/128][32][4]  (their scales per 32-row quarter
//                               t32 of a tile (padded row / 32), k-step and
//                               row, as for hs below);
//   The down GEMM's A operand h, per 32-row quarter t32 of a tile (padded
//   row / 32) and k-step j (4 blocks = 128 codes):
//   hq int8 [4*T_bound][KBMAX/4][32 rows][128]  (a 4 KiB slab per (t32, j);
//                               the 16-code piece p of row r (block p/2 of the
//                               k-step, half p%2) sits at byte 16 * (p ^ (r % 8))
//                               of the row's 128-byte line);
//   hs fp16 [4*T_bound][KBMAX/4][32][4]         (their scales);
//   partial fp32 [N][k + has_shared][d].
// The decode region, always reserved for Nd = min(N, DECODE_MAX_TOKENS) tokens
// (so the total never shrinks as N grows), used by decode calls only:
//   dlist i32 [4 + 16 * (min(E, Nd*k) + has_shared)]  (dlist[0] = number of
//                               active groups; entry a = dlist + 4 + 16 a:
//                               {group, rows c, 6 unused, pair p[8]}, where
//                               row j < c is the (token, slot) pair
//                               p = token * kk + slot, tokens ascending;
//                               routed groups ascending, then the shared one);
//   dxq int8 [Nd][d_pad], dxs fp16 [Nd][d_pad/32]   (token-major activation
//                               codes/scales, zero past d);
//   dhq int8 [Nd*kk][kmax_pad], dhs fp16 [Nd*kk][kmax_pad/32]  (h per pair).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_ffn.h"

namespace moe {

constexpr int QB = 32;            // int8 block length (Q8_0 / activation blocks)
constexpr int Q8_BYTES = 34;      // Q8_0 block: binary16 scale + 32 codes
constexpr int KPAD = 128;         // K-dimension padding granule (4 blocks)
constexpr int ROUTE_TILE = 8;     // tokens per routing workgroup
constexpr int MT_WG = 128;        // rows per grouped-GEMM workgroup tile
constexpr int MT_WAVE = 32;       // rows per wavefront
constexpr int GU_COLS = 64;       // SwiGLU output columns per gate/up strip
constexpr int DN_COLS = 128;      // output columns per down strip
constexpr int KSTEP = 4;          // 32-blocks per GEMM k-step
constexpr int KSTEP_BYTES = 17 * 1024;     // gate/up k-step: codes (16 KiB) + scales (1 KiB)
constexpr int DN_KSTEP_BYTES = 18 * 1024;  // down k-step: codes (16 KiB) + scale pairs (2 KiB)
constexpr int Q4K_VALUES = 256;            // weights per Q4_K super-block
constexpr int Q4K_BYTES = 144;             // Q4_K super-block: d, dmin, 12 scale/min bytes, 128 code bytes
constexpr int Q4K_KSTEP_BYTES = 12 * 1024; // Q4_K k-step (gate/up and down): codes 8 KiB + D and M pairs 2 KiB each
constexpr int Q3K_BYTES = 110;             // Q3_K super-block: 32 high-bit bytes, 64 code bytes, 12 scale bytes, d
constexpr int MAX_TOPK = 16;
constexpr int MAX_EXPERTS = 256;
constexpr int DECODE_MAX_TOKENS = 8;
constexpr int DLIST_ENTRY = 16;   // ints per decode active-group entry
constexpr int DLIST_PAIRS = 8;    // offset of the pair list in an entry

struct Dims {
  int d, E, k, F, Fs, norm;
  int has_shared;
  int d_pad, F_pad, Fs_pad, kmax_pad;  // kmax_pad = max(F_pad, Fs_pad)
  int E64;
  int G;  // expert groups = E + has_shared
};

inline int round_up(int v, int m) { return (v + m - 1) / m * m; }

struct WsLayout {
  size_t logits, ids, rank, w, gs, hist, exp_start, tok_i, tok_k, row_tok, tiles, gq, gxs, gqs, hq, hs, partial;
  size_t dlist, dxq, dxs, dhq, dhs;  // decode region (min(N, 8) tokens)
  size_t total;
  int n_route_tiles;
  int tile_bound;
};

WsLayout ws_layout(const Dims& dm, int max_tokens);

}  // namespace moe

struct moe_ffn_weights {
  moe_ffn_dims user;
  moe::Dims dm;
  int device;
  int has_bias;
  void* base;  // one allocation holding every plane below
  float* router_wt;
  float* router_bias;
  float* sh_gate_vec;
  uint8_t* gu;
  uint8_t* dn;
  uint8_t* sh_gu;
  uint8_t* sh_dn;
  int32_t* dn_exp;  // [G] exponent e of each group's down scale plane
  int fmt;          // format of the planes: MOE_FFN_FMT_Q8_0 (also for Q3_K rows) or MOE_FFN_FMT_Q4_K
  int n_cu;         // compute units of the device
  size_t gu_per_expert, dn_per_expert;  // bytes
};

namespace moe {

// ---- launchers (each returns hipGetLastError() of its launch) ----
// Gate/up form (dn_exp == NULL, 17 KiB k-steps) or down form (dn_exp = the
// groups' exponents, 18 KiB k-steps with scale pairs).
hipError_t launch_repack_q8(const uint8_t* src0, const uint8_t* src1, int n_groups,
                            size_t src_group_bytes, int src_rows, int src_blocks, int tiles_per_src,
                            int n_strips, int kb_pad, uint8_t* dst, size_t dst_group_bytes,
                            const int32_t* dn_exp, hipStream_t s);
// e[g] = the smallest e >= 0 with |scale| * 2^(23 - e) <= 65504 for every Q8_0
// block of group g (n_groups groups of n_blocks blocks, src_group_bytes apart).
// Q4_K rows (super-blocks of 144 bytes, src_supers per row) to the Q4_K
// planes: n_strips strips of n_ksteps k-steps per group; tiles_per_src as for
// launch_repack_q8.  *overflow (device) is set to 1 when a finite sub-block
// scale or min d * sc or dmin * m exceeds the binary16 range.
hipError_t launch_repack_q4k(const uint8_t* src0, const uint8_t* src1, int n_groups, size_t src_group_bytes,
                             int src_rows, int src_supers, int tiles_per_src, int n_strips, int n_ksteps,
                             uint8_t* dst, size_t dst_group_bytes, int32_t* overflow, hipStream_t s);
// Q3_K rows (supers super-blocks per row, rows rows per group) to Q8_0 rows
// with the same values exactly: per 32-block scale -d and codes
// -(sc - 32) * q (dst holds n_groups * rows * supers * 8 blocks of 34 bytes).
hipError_t launch_q3k_to_q8(const uint8_t* src, int n_groups, size_t src_group_bytes, int rows, int supers,
                            uint8_t* dst, size_t dst_group_bytes, hipStream_t s);
hipError_t launch_scale_exponent(const uint8_t* src, int n_groups, size_t src_group_bytes,
                                 long n_blocks, int32_t* e, hipStream_t s);
hipError_t launch_transpose_router(const float* w, int E, int d, int E64, float* wt, hipStream_t s);

// n_cu: compute units of the device (a grid larger than one workgroup per CU
// takes the router form that fits two per CU).
hipError_t launch_router(const float* x, int n, int d, const float* wt, const float* bias, int E,
                         int E64, float* logits, int n_cu, hipStream_t s);
// Router and routing in one launch (E <= 64): ids, w, rank and the tile
// histograms as launch_route writes them; no logits in global memory.
hipError_t launch_router_route(const float* x, int n, int d, const float* wt, const float* bias,
                               int E, int k, int norm, int32_t* ids, float* w, int32_t* rank,
                               int32_t* hist, int n_cu, hipStream_t s);
// Token-major activation quantiser: every row of x [n][d] quantised per
// 32-block into xq [n][d_pad] / xs [n][d_pad/32] (zero past d), optionally
// also into xq_out [n][d] / xs_out [n][d/32]; with shg != NULL also
// gs[t] = sigmoid(x[t] . shg).
struct RowQuant {
  const float* x;
  int d, d_pad;
  const float* shg;
  float* gs;
  int8_t* xq;
  uint16_t* xs;
  int8_t* xq_out;
  uint16_t* xs_out;
};
// Routing from the logits (E > 64), in the same launch as the token-major
// quantiser rq (its workgroups run beside the routing ones).
hipError_t launch_route(const float* logits, int n, int E, int k, int norm, int32_t* ids, float* w,
                        int32_t* rank, int32_t* hist, const RowQuant& rq, hipStream_t s);
hipError_t launch_quantize(const float* v, int64_t n_values, int8_t* q, uint16_t* scales,
                           hipStream_t s);
// The bucketing (expStart, expTokI/expTokK, the tile table and its row
// tokens row_tok [T_bound][128]) and, in the same
// workgroups, the activation quantiser: every token row quantised per
// 32-block, codes into gq [N][d_pad], scales into gqs at each of the token's
// tile rows (zero past d); with
// sh_gate_vec != NULL also gs[t] = sigmoid(x[t] . g); xq_out [N][d] /
// xs_out [N][d/32] (each optional) receive copies of the unpadded width.
// With xs_tok != NULL the codes, the gate and the optional copies were
// written by the routing launch (RowQuant, scales xs_tok [N][d_pad/32]): the
// workgroups only place the scales at the tile rows, and x is not read.
hipError_t launch_bucket_quantize(const int32_t* ids, const int32_t* rank, const int32_t* hist, int n,
                                  int E, int k, int has_shared, int32_t* exp_start, int32_t* tok_i,
                                  int32_t* tok_k, int32_t* row_tok, int32_t* tiles, int tile_bound,
                                  const float* x, int d, int d_pad, int8_t* gq, uint16_t* gqs,
                                  const float* sh_gate_vec, float* gs, int8_t* xq_out, uint16_t* xs_out,
                                  const uint16_t* xs_tok, hipStream_t s);

struct GemmArgs {
  // common
  const int32_t* tiles;
  const int32_t* tok_i;
  const int32_t* tok_k;
  const int32_t* row_tok;  // [T_bound][128]: the token of each tile row
  int E;
  int G;          // groups: E routed (+1 shared)
  int n_tokens;
  int p_total;    // CSR rows: N*k (+N)
  int tile_bound;
  int kbmax;  // kmax_pad / 32
  int8_t* hq;
  uint16_t* hs;
  // gate/up
  const int8_t* gq;
  const uint16_t* gqs;
  int d_pad;
  const uint8_t* gu;
  size_t gu_group;
  const uint8_t* sh_gu;
  int F_pad, Fs_pad;
  // down
  const uint8_t* dn;
  size_t dn_group;
  const uint8_t* sh_dn;
  const int32_t* dn_exp;
  float* partial;
  int d;
  int kk;
  int reverse;  // 1: walk the tile table from its last tile (serpentine chunk order)
};

hipError_t launch_gateup(const GemmArgs& a, hipStream_t s);
hipError_t launch_down(const GemmArgs& a, hipStream_t s);
// The same two GEMMs on Q4_K weight planes.
hipError_t launch_gateup_q4k(const GemmArgs& a, hipStream_t s);
hipError_t launch_down_q4k(const GemmArgs& a, hipStream_t s);
// One k-block of one (tile, strip) of a grouped GEMM through the product's
// copies, LDS layout and int8 MFMA: exact int32 block sums [128][128], the A
// codes [128][32] and {group, row0, row_end, n_tiles} (one workgroup).
hipError_t launch_block_sums(const GemmArgs& a, bool gateup, int tile, int strip, int kblock, int32_t* sums,
                             int8_t* acodes, int32_t* info, hipStream_t s);

// ---- decode (1 <= N <= DECODE_MAX_TOKENS) ----
// Router logits [N][E] (the same fp32 block order as launch_router), plus the
// token-major activation codes dxq/dxs (row strides d_pad and d_pad/32, zero
// past d) and, with sh_gate_vec != NULL, gs[t] = sigmoid(x[t] . g).
hipError_t launch_decode_router(const float* x, int n, int d, int d_pad, const float* wt,
                                const float* bias, int E, int E64, float* logits,
                                const float* sh_gate_vec, float* gs, int8_t* dxq, uint16_t* dxs,
                                hipStream_t s);
// The decode matvecs.  The gate/up launch also routes: every workgroup
// derives the top-k of the N tokens from the logits and so its own group and
// (token, slot) pairs; workgroup 0 writes ids, w, the CSR and dlist, which
// the down launch reads.
struct DecodeArgs {
  // routing (gate/up launch)
  const float* logits;  // [N][E]
  int n, k, norm, has_shared;
  int32_t* ids;
  float* w;
  int32_t* exp_start;
  int32_t* tok_i;
  int32_t* tok_k;
  int32_t* dlist;  // written by the gate/up launch, read by the down launch
  int E, kk, n_bound;  // n_bound: upper bound on the number of active groups
  int n_cu;            // compute units of the device (the matvec grids are sized to what is resident)
  // gate/up: A = dxq/dxs rows of the pairs' tokens
  const int8_t* xq;
  const uint16_t* xs;
  const uint8_t* gu;
  size_t gu_group;
  const uint8_t* sh_gu;
  int d, d_pad, F_pad, Fs_pad, kmax_pad;
  int8_t* hq;
  uint16_t* hs;
  // down: A = hq/hs rows of the pairs, output partial[pair][d]
  const uint8_t* dn;
  size_t dn_group;
  const uint8_t* sh_dn;
  const int32_t* dn_exp;
  float* partial;
};
hipError_t launch_decode_gateup(const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_down(const DecodeArgs& a, hipStream_t s);
// One token (n == 1) with at most 9 slots (k plus the shared expert): the down
// matvec and the ordered combine in one launch, out [d] and partial as the
// two launches write them.
constexpr int DECODE_FUSED_MAX_SLOTS = 9;
hipError_t launch_decode_down_combine(const DecodeArgs& a, const float* gs, float* out, hipStream_t s);

hipError_t launch_combine(const float* partial, const float* w, const float* gs, int n, int k,
                          int kk, int d, float* out, hipStream_t s);
hipError_t launch_combine_residual_rmsnorm(const float* partial, const float* w, const float* gs, int n,
                                           int k, int kk, int d, float* h, float* xn, float eps,
                                           hipStream_t s);
hipError_t launch_residual_rmsnorm(float* h, const float* y, float* xn, int n, int d, float eps,
                                   hipStream_t s);

}  // namespace moe
