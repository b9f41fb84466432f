// decode.hip -- the decode-time expert matvecs (1 <= N <= 8 tokens).
//
// SharpInference #408 "Hypothesis" lever 1: at decode the expert FFN is eight
// small matvecs per token, launched one by one; the lever is one gathered
// launch per stage over the selected experts, each expert's weights read once
// for all the tokens that picked it.  With at most 8 rows per expert the
// grouped GEMM's 32-row MFMA tiles would be mostly padding and its per-tile
// prologue dominates, so these kernels are matvecs on the int8 dot unit
// (v_dot4_i32_i8) that stream the weights straight into registers:
//
// * Routing: the gate/up launch derives the top-k of its N tokens itself in
//   every workgroup (from the N x E logits: a few microseconds less than a
//   launch of its own); its workgroup 0 writes the routing outputs and the
//   group list the down launch reads.
// * Unit of work: one active group (routed experts ascending, then the
//   shared expert) and 32
//   output columns: a gate/up unit is one SwiGLU block of 32 h columns (gate
//   tile + up tile of the same strip), a down unit two 32-row tiles of the
//   down matrix.  Both read the planes the grouped GEMMs read (no second copy
//   of the weights): per k-step 8 chunks of 1 KiB, lane l holding row l%32 and
//   codes [16 (l/32), +16) of each 32-block.
// * The 8 wavefronts of a workgroup split the k-steps (wavefront w takes
//   k-steps w and w+8 of each pass of 16), requesting both before it waits
//   for either: a workgroup has its whole 128 KiB share in flight at once.  The group's activation rows (<= 8) are staged in LDS
//   per pass of up to DPK k-steps; a lane reads its 16 codes of each block
//   there (two distinct addresses per read: a broadcast).
// * Per block, row and token: exact int32 dot of the lane's 16 codes, then
//   acc += float(dot) * (sw * sa), where sw * sa is exact in fp32 (two
//   binary16 values).  The two half-block partial sums of a row meet in the
//   final reduction (over the lane pair, then the 8 wavefronts in order).
// * Gate/up epilogue: h = silu(gate) * up and its per-32 requantisation
//   (the decisions of quant_block32, one block per token) into the pair's h
//   row; down epilogue: times 2^(e - 23) (the down plane stores W =
//   sw * 2^(23 - e)) into partial[pair].
#include <algorithm>

#include "device_util.h"
#include "route_util.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int DW = 8;                  // wavefronts per workgroup
constexpr int DPK = 16;                // k-steps per staged activation pass
constexpr int ACT_BYTES = DECODE_MAX_TOKENS * DPK * 128;            // 16 KiB of codes
constexpr int ACS_BYTES = DECODE_MAX_TOKENS * DPK * KSTEP * 2;      // 1 KiB of scales
constexpr int RED_BYTES = DW * 2 * DECODE_MAX_TOKENS * 32 * 4;      // 16 KiB reduction
constexpr int DEC_LDS = (ACT_BYTES + ACS_BYTES > RED_BYTES) ? ACT_BYTES + ACS_BYTES : RED_BYTES;

// One k-step of a unit for this lane: codes of blocks kbi = 0..3 for the two
// tiles, and the scales of the lane's row in both tiles (gate/up: 4 binary16
// scales per tile; down: two {W, W/2} pair words per tile, blocks 0-1 and 2-3).
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
struct Piece {
  v4u w[KSTEP][2];
  v2u s[2][2];
};

// The weights are read with buffer loads: one resource over the unit's strip
// (SGPRs), the per-chunk byte offset in an SGPR and the lane's offset in one
// VGPR that never changes, so no load ever waits to reuse an address register
// of a load still in flight (with 64-bit VGPR addresses the second k-step's
// loads did).  The range check is off (num_records = 2^32 - 1): every offset
// is inside the strip by construction.
constexpr int BUF_DWORD3 = 0x00020000;  // raw buffer, 32-bit data format

template <bool GATEUP>
__device__ __forceinline__ void load_piece(__amdgpu_buffer_rsrc_t rs, int step_off, int tsel0, int tstride,
                                           uint32_t o_code, uint32_t o_scale, Piece& p) {
#pragma unroll
  for (int kbi = 0; kbi < KSTEP; ++kbi)
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
      p.w[kbi][ti] = __builtin_amdgcn_raw_buffer_load_b128(rs, o_code, step_off + (kbi * 4 + tsel0 + tstride * ti) * 1024, 0);
    }
#pragma unroll
  for (int ti = 0; ti < 2; ++ti) {
    const int tt = tsel0 + tstride * ti;
    if constexpr (GATEUP) {
      p.s[ti][0] = __builtin_amdgcn_raw_buffer_load_b64(rs, o_scale, step_off + 16 * 1024 + tt * 256, 0);
      p.s[ti][1] = p.s[ti][0];
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        p.s[ti][h] = __builtin_amdgcn_raw_buffer_load_b64(rs, o_scale, step_off + 16 * 1024 + tt * 512 + h * 256, 0);
      }
    }
  }
}

// Force the arguments a kernel uses into SGPRs at this point (the entry
// block), in one statement, so that they are fetched as one batch of scalar
// loads.
template <bool GATEUP>
__device__ __forceinline__ void pin_args(const DecodeArgs& a) {
  // input operands only: the code below keeps using the fields themselves
  if constexpr (GATEUP)
    asm volatile("" ::"s"(a.logits), "s"(a.n), "s"(a.k), "s"(a.has_shared), "s"(a.E), "s"(a.kk), "s"(a.xq),
                 "s"(a.xs), "s"(a.gu), "s"(a.gu_group), "s"(a.sh_gu), "s"(a.d_pad), "s"(a.F_pad), "s"(a.Fs_pad),
                 "s"(a.kmax_pad), "s"(a.hq), "s"(a.hs));
  else
    asm volatile("" ::"s"(a.dlist), "s"(a.E), "s"(a.n_bound), "s"(a.d), "s"(a.d_pad), "s"(a.F_pad),
                 "s"(a.Fs_pad), "s"(a.kmax_pad), "s"(a.hq), "s"(a.hs), "s"(a.dn), "s"(a.dn_group),
                 "s"(a.sh_dn), "s"(a.dn_exp), "s"(a.partial));
}

// pr[j] for a per-lane j (the pairs sit in lanes 0..c-1 of one register)
__device__ __forceinline__ int pick(int tbl, int j) { return __shfl(tbl, j, 64); }

__device__ __forceinline__ float h2f(uint32_t bits16) {
  return __half2float(__ushort_as_half((uint16_t)(bits16 & 0xffffu)));
}

// The piece's contribution for every staged row j < c: act = the k-step's
// 128 codes of the staged rows (row stride DPK * 128), as = their scales.
template <bool GATEUP>
__device__ __forceinline__ void compute_piece(const Piece& p, const int8_t* act, const uint16_t* as, int c,
                                              int lane, float (&acc)[2][DECODE_MAX_TOKENS]) {
  float sw[2][KSTEP];
#pragma unroll
  for (int ti = 0; ti < 2; ++ti) {
    if constexpr (GATEUP) {
      sw[ti][0] = h2f(p.s[ti][0][0]);
      sw[ti][1] = h2f(p.s[ti][0][0] >> 16);
      sw[ti][2] = h2f(p.s[ti][0][1]);
      sw[ti][3] = h2f(p.s[ti][0][1] >> 16);
    } else {  // W of blocks 2h, 2h+1: the low halves of the two pair words
      sw[ti][0] = h2f(p.s[ti][0][0]);
      sw[ti][1] = h2f(p.s[ti][0][1]);
      sw[ti][2] = h2f(p.s[ti][1][0]);
      sw[ti][3] = h2f(p.s[ti][1][1]);
    }
  }
  const int half = lane >> 5;
#pragma unroll
  for (int j = 0; j < DECODE_MAX_TOKENS; ++j) {
    if (j < c) {  // workgroup-uniform
      const int8_t* arow = act + j * (DPK * 128) + half * 16;
      uint4 av[KSTEP];
#pragma unroll
      for (int kbi = 0; kbi < KSTEP; ++kbi) av[kbi] = *reinterpret_cast<const uint4*>(arow + kbi * 32);
      const uint2 s2 = *reinterpret_cast<const uint2*>(as + j * (DPK * KSTEP));
      const float sa[KSTEP] = {h2f(s2.x), h2f(s2.x >> 16), h2f(s2.y), h2f(s2.y >> 16)};
#pragma unroll
      for (int kbi = 0; kbi < KSTEP; ++kbi)
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) {
          const v4u wv = p.w[kbi][ti];
          int dot = __builtin_amdgcn_sdot4((int)wv[0], (int)av[kbi].x, 0, false);
          dot = __builtin_amdgcn_sdot4((int)wv[1], (int)av[kbi].y, dot, false);
          dot = __builtin_amdgcn_sdot4((int)wv[2], (int)av[kbi].z, dot, false);
          dot = __builtin_amdgcn_sdot4((int)wv[3], (int)av[kbi].w, dot, false);
          acc[ti][j] = __builtin_fmaf((float)dot, sw[ti][kbi] * sa[kbi], acc[ti][j]);
        }
    }
  }
}

// ---- routing inside the gate/up launch ----
// The routing state of one workgroup: for every token the slot of each expert
// (0xff: not picked), the picked experts in slot order and their logits.
struct DecRoute {
  uint8_t slot[DECODE_MAX_TOKENS][MAX_EXPERTS];
  int sel[DECODE_MAX_TOKENS][MAX_TOPK];
  float selv[DECODE_MAX_TOKENS][MAX_TOPK];
  int wtot[4];
  __attribute__((aligned(16))) unsigned long long kl[DECODE_MAX_TOKENS][64];  // E <= 64: each token's keys, for wave_key_rank
};
// The active groups in list order (routed experts ascending, then the shared
// expert): group id, row count and the rows' (token, slot) pairs.
constexpr int MAX_GROUPS = DECODE_MAX_TOKENS * MAX_TOPK + 1;
struct GroupList {
  int g[MAX_GROUPS];
  int c[MAX_GROUPS];
  int pairs[MAX_GROUPS][DECODE_MAX_TOKENS];
};

// Inclusive prefix sum over the wavefront (same DPP pattern with additions).
__device__ __forceinline__ int wave_inclusive_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Route the N <= 8 tokens from their logits (every workgroup of the launch
// does this; the top-k of the contract: logit descending, then id
// ascending, by the same 64-bit keys as the prefill routing).  Wavefront t
// takes token t's k largest keys one at a time (a wavefront maximum per
// slot: of the high words, then of the low words among the lanes that hold
// that high word).  Thread e then counts the tokens that picked expert e; one
// scan gives each active expert its index in the group list and its CSR
// start.  Fills GL and returns the number of groups.  Workgroup 0 also writes
// ids, w (softmax over all E, then the optional renormalisation over the k
// slots), expStart/expTokI/expTokK and the group list the down launch reads.
__device__ __forceinline__ int decode_route(const DecodeArgs& a, DecRoute& R, GroupList& GL, int wave, int lane) {
  const int n = a.n, E = a.E, k = a.k, kk = a.kk, tid = threadIdx.x;
  const bool wg0 = blockIdx.x == 0;
  if (wave < n) {
    float lv[4];
    unsigned long long kv[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) lv[m] = a.logits[(size_t)wave * E + min(lane + 64 * m, E - 1)];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int e = lane + 64 * m;
      kv[m] = e < E ? topk_key(lv[m], e) : 0ull;  // every real key is > 0
      R.slot[wave][e] = 0xff;
    }
    if (E <= 64) {
      // one key per lane: its rank is its slot (keys are distinct)
      const int rk = wave_key_rank(kv[0], R.kl[wave], lane);
      if (lane < E && rk < k) {
        R.slot[wave][lane] = (uint8_t)rk;
        R.selv[wave][rk] = lv[0];
        R.sel[wave][rk] = lane;
      }
    } else {
      for (int s = 0; s < k; ++s) {
        unsigned long long b = kv[0];
#pragma unroll
        for (int m = 1; m < 4; ++m) b = kv[m] > b ? kv[m] : b;
        const unsigned long long mx = wave_max_key(b);
        const uint32_t ml = (uint32_t)mx;
#pragma unroll
        for (int m = 0; m < 4; ++m)
          if (kv[m] == mx) {  // keys are distinct: one lane, one m
            R.slot[wave][lane + 64 * m] = (uint8_t)s;
            R.selv[wave][s] = lv[m];
            kv[m] = 0ull;
          }
        if (lane == 0) R.sel[wave][s] = (int)~ml;
      }
    }
    if (wg0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const float m0 = R.selv[wave][0];
      float part = 0.0f;
#pragma unroll
      for (int m = 0; m < 4; ++m)
        if (lane + 64 * m < E) part += expf(lv[m] - m0);
      part = wave_sum_f32(part);
      float p = lane < k ? expf(R.selv[wave][min(lane, MAX_TOPK - 1)] - m0) / part : 0.0f;
      if (a.norm) p = p / wave_sum_f32(p);
      if (lane < k) {
        a.ids[(size_t)wave * k + lane] = R.sel[wave][lane];
        a.w[(size_t)wave * k + lane] = p;
      }
    }
  }
  __syncthreads();
  // thread e < E: its token count (low 16 bits) and active flag (high 16),
  // exclusive-scanned over the first four wavefronts together
  int cnt = 0;
  if (tid < E)
    for (int t = 0; t < n; ++t) cnt += R.slot[t][tid] != 0xff ? 1 : 0;
  const int v = cnt | ((cnt > 0 ? 1 : 0) << 16);
  const int inc = wave_inclusive_sum(v);
  if (lane == 63 && wave < 4) R.wtot[wave] = inc;
  __syncthreads();
  int pre = 0;
  for (int w2 = 0; w2 < min(wave, 4); ++w2) pre += R.wtot[w2];
  const int ex = pre + inc - v;
  const int n_act = (R.wtot[0] + R.wtot[1] + R.wtot[2] + R.wtot[3]) >> 16;
  const int start = ex & 0xffff, aidx = ex >> 16;
  const int P = n * k;
  if (tid < E && cnt > 0) {
    GL.g[aidx] = tid;
    GL.c[aidx] = cnt;
    int32_t* ent = a.dlist + 4 + DLIST_ENTRY * aidx;
    if (wg0) {
      ent[0] = tid;
      ent[1] = cnt;
    }
    int j = 0;
    for (int t = 0; t < n; ++t) {
      const int s = R.slot[t][tid];
      if (s != 0xff) {
        GL.pairs[aidx][j] = t * kk + s;
        if (wg0) {
          ent[DLIST_PAIRS + j] = t * kk + s;
          a.tok_i[start + j] = t;
          a.tok_k[start + j] = s;
        }
        ++j;
      }
    }
  }
  if (a.has_shared) {
    if (tid == 0) {
      GL.g[n_act] = E;
      GL.c[n_act] = n;
    }
    if (tid < n) GL.pairs[n_act][tid] = tid * kk + k;
  }
  if (wg0) {
    if (tid < E) a.exp_start[tid] = start;
    if (tid == 0) {
      a.exp_start[E] = P;
      if (a.has_shared) a.exp_start[E + 1] = P + n;
      a.dlist[0] = n_act + a.has_shared;
    }
    if (a.has_shared) {
      int32_t* ent = a.dlist + 4 + DLIST_ENTRY * n_act;
      if (tid == 0) {
        ent[0] = E;
        ent[1] = n;
      }
      if (tid < n) {
        ent[DLIST_PAIRS + tid] = tid * kk + k;
        a.tok_i[P + tid] = tid;
        a.tok_k[P + tid] = k;
      }
    }
  }
  __syncthreads();
  return n_act + a.has_shared;
}

// The group list the gate/up launch wrote, copied into LDS (its count and
// all entries in one round trip: the entries read past the count stay
// inside the list's n_bound entries and are not used).
__device__ __forceinline__ int load_group_list(const DecodeArgs& a, GroupList& GL) {
  const int tid = threadIdx.x;
  const int n_groups = min(a.dlist[0], a.n_bound);
  for (int q = tid; q < a.n_bound * DLIST_ENTRY; q += DW * 64) {
    const int ei = q / DLIST_ENTRY, f = q - ei * DLIST_ENTRY;
    const int v = a.dlist[4 + q];
    if (f == 0) GL.g[ei] = v;
    else if (f == 1) GL.c[ei] = min(max(v, 1), DECODE_MAX_TOKENS);
    else if (f >= DLIST_PAIRS) GL.pairs[ei][f - DLIST_PAIRS] = v;
  }
  __syncthreads();
  return n_groups;
}

// GATEUP: unit u = (strip u/2, tile pair u%2) of the [gate;up] plane, columns
// 32u .. 32u+31 of h.  !GATEUP: unit u = (strip u/2, tiles 2(u%2), 2(u%2)+1)
// of the down plane, output rows 64u .. 64u+63.  A workgroup takes units
// blockIdx.x, + gridDim.x, ... of the (group, unit) list, so that the routing
// (or the list) is read once per workgroup and no workgroup is surplus.
template <bool GATEUP>
__global__ __launch_bounds__(DW * 64) void decode_gemv_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[DEC_LDS];
  __shared__ GroupList GL;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Start-up latency is the cost that matters for a kernel of a few
  // workgroups per CU: every argument is requested at once (one scalar round
  // trip, not one per branch that first needs a field); then the routing
  // input (gate/up: the logits; down: the group list) in one more.
  pin_args<GATEUP>(a);
  const int units = GATEUP ? a.kmax_pad / 32 : a.d_pad / 64;
  int n_groups;
  if constexpr (GATEUP) {
    __shared__ DecRoute R;
    n_groups = decode_route(a, R, GL, wave, lane);
  } else {
    n_groups = load_group_list(a, GL);
  }
  const int total = n_groups * units;
  const uint32_t o_code = (uint32_t)lane * 16, o_scale = (uint32_t)(lane & 31) * 8;
  int8_t* s_act = reinterpret_cast<int8_t*>(lds);
  uint16_t* s_as = reinterpret_cast<uint16_t*>(lds + ACT_BYTES);
  float* red = reinterpret_cast<float*>(lds);

  for (int id = blockIdx.x; id < total; id += gridDim.x) {
    const int ei = id / units, u = id - ei * units;
    const int g = __builtin_amdgcn_readfirstlane(GL.g[ei]);
    const int c = __builtin_amdgcn_readfirstlane(GL.c[ei]);
    if (g < 0 || g > a.E || c < 1 || c > DECODE_MAX_TOKENS) continue;
    const bool shared = g == a.E;
    if (shared && !(GATEUP ? a.sh_gu : a.sh_dn)) continue;
    const int Fg_pad = shared ? a.Fs_pad : a.F_pad;
    if (GATEUP && u * 32 >= Fg_pad) continue;
    // the rows' (token, slot) pairs in lanes 0..c-1
    const int pr = GL.pairs[ei][min(lane, c - 1)];

    const int KS = (GATEUP ? a.d_pad : Fg_pad) / (KSTEP * QB);
    const int step_bytes = GATEUP ? KSTEP_BYTES : DN_KSTEP_BYTES;
    const uint8_t* plane = GATEUP ? (shared ? a.sh_gu : a.gu + (size_t)g * a.gu_group)
                                  : (shared ? a.sh_dn : a.dn + (size_t)g * a.dn_group);
    plane += (size_t)(u >> 1) * KS * step_bytes;
    const int tsel0 = GATEUP ? (u & 1) : 2 * (u & 1);  // first tile; the second is +2 (up) or +1
    const int tstride = GATEUP ? 2 : 1;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(plane), (short)0, -1, BUF_DWORD3);

    float acc[2][DECODE_MAX_TOKENS];
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int j = 0; j < DECODE_MAX_TOKENS; ++j) acc[ti][j] = 0.0f;

    // Per pass of DPK = 2 * DW k-steps, wavefront w computes k-steps ks0 + w
    // and ks0 + w + DW; both are requested before the activations are staged,
    // so each wavefront has its whole share of the pass in flight at once.
    static_assert(DPK == 2 * DW, "two k-steps per wavefront and pass");
    static_assert(DECODE_MAX_TOKENS * DPK * 8 <= 2 * DW * 64, "two 16-byte activation pieces per thread");
    static_assert(DECODE_MAX_TOKENS * DPK <= DW * 64, "one scale word per thread");
    for (int ks0 = 0; ks0 < KS; ks0 += DPK) {
      const int ks_end = min(ks0 + DPK, KS), npk = ks_end - ks0;
      const int k0 = ks0 + wave, k1 = ks0 + wave + DW;
      // The pass's activation rows (codes [j][npk * 128], scales [j][npk * 4];
      // at most 2 x 512 16-byte pieces and 128 scale words) are requested
      // first: they hit in the caches, and waiting for them then does not
      // wait for the weights requested after them.  Addresses are clamped
      // into the rows (unconditional loads), the LDS writes masked.
      const int nq = c * npk * 8, ns = c * npk;
      auto code_src = [&](int q) {
        q = min(q, nq - 1);
        const int j = q / (npk * 8), o = q - j * (npk * 8);
        const int prj = pick(pr, j);
        return GATEUP ? reinterpret_cast<const uint4*>(a.xq + (size_t)(prj / a.kk) * a.d_pad + ks0 * 128) + o
                      : reinterpret_cast<const uint4*>(a.hq + (size_t)prj * a.kmax_pad + ks0 * 128) + o;
      };
      const int q0 = threadIdx.x, q1 = threadIdx.x + DW * 64;
      const uint4 c0 = *code_src(q0), c1 = *code_src(q1);
      const int qs = min((int)threadIdx.x, ns - 1), js = qs / npk, os = qs - js * npk;
      const int prs = pick(pr, js);
      const uint2 sv = GATEUP
          ? reinterpret_cast<const uint2*>(a.xs + (size_t)(prs / a.kk) * (a.d_pad / QB) + ks0 * KSTEP)[os]
          : reinterpret_cast<const uint2*>(a.hs + (size_t)prs * (a.kmax_pad / QB) + ks0 * KSTEP)[os];
      // both k-steps requested unconditionally (a k-step past the pass
      // re-reads the pass's last one and is not computed): no branch between
      // requests
      Piece p0, p1;
      load_piece<GATEUP>(rs, min(k0, ks_end - 1) * step_bytes, tsel0, tstride, o_code, o_scale, p0);
      load_piece<GATEUP>(rs, min(k1, ks_end - 1) * step_bytes, tsel0, tstride, o_code, o_scale, p1);
      __builtin_amdgcn_sched_barrier(0);  // every request is out before any wait
      lds_barrier();  // every wavefront is done with the LDS of the previous pass or unit
      if (q0 < nq) reinterpret_cast<uint4*>(s_act + (q0 / (npk * 8)) * (DPK * 128))[q0 % (npk * 8)] = c0;
      if (q1 < nq) reinterpret_cast<uint4*>(s_act + (q1 / (npk * 8)) * (DPK * 128))[q1 % (npk * 8)] = c1;
      if ((int)threadIdx.x < ns) reinterpret_cast<uint2*>(s_as + js * (DPK * KSTEP))[os] = sv;
      lds_barrier();
      if (k0 < ks_end) compute_piece<GATEUP>(p0, s_act + (k0 - ks0) * 128, s_as + (k0 - ks0) * KSTEP, c, lane, acc);
      if (k1 < ks_end) compute_piece<GATEUP>(p1, s_act + (k1 - ks0) * 128, s_as + (k1 - ks0) * KSTEP, c, lane, acc);
    }

    // Reduction: the lane pair (two halves of each block), then the
    // wavefronts in order.  red[w][ti][j][r] reuses the staging buffer.
    lds_barrier();
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int j = 0; j < DECODE_MAX_TOKENS; ++j) {
        if (j < c) {
          const float v = acc[ti][j] + __shfl_xor(acc[ti][j], 32, 64);
          if (lane < 32) red[((wave * 2 + ti) * DECODE_MAX_TOKENS + j) * 32 + lane] = v;
        }
      }
    lds_barrier();
    const int tid = threadIdx.x;
    if constexpr (GATEUP) {
      // thread (j = tid / 32, r = tid % 32): column 32u + r of h for row j;
      // a row's 32 threads are one half-wavefront (the quantiser's exchanges
      // stay inside it)
      const int j = tid >> 5, r = tid & 31;
      if (tid < DECODE_MAX_TOKENS * 32 && j < c) {
        float gv = 0.0f, uv = 0.0f;
#pragma unroll
        for (int w = 0; w < DW; ++w) {
          gv += red[((w * 2 + 0) * DECODE_MAX_TOKENS + j) * 32 + r];
          uv += red[((w * 2 + 1) * DECODE_MAX_TOKENS + j) * 32 + r];
        }
        const float h = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
        int8_t q;
        uint16_t s16;
        quant_block32(h, q, s16);
        const int prj = pick(pr, j);
        a.hq[(size_t)prj * a.kmax_pad + u * 32 + r] = q;
        if (r == 0) a.hs[(size_t)prj * (a.kmax_pad / QB) + u] = s16;
      }
    } else {
      // thread (ti, j, r): output row 64u + 32 ti + r of pair row j
      const int ti = tid >> 8, j = (tid >> 5) & 7, r = tid & 31;
      const int row = 64 * u + 32 * ti + r;
      const int prj = pick(pr, j);
      if (j < c && row < a.d) {
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < DW; ++w) v += red[((w * 2 + ti) * DECODE_MAX_TOKENS + j) * 32 + r];
        const int eg = a.dn_exp[g];
        a.partial[(size_t)prj * a.d + row] = ldexpf(v, eg - 23);
      }
    }
  }
}

// ---- down matvec + ordered combine for one token ----
// Decode of a single token (n == 1, kk = k (+1) <= DC_SB slots): the down
// matvec of its selected experts (and the shared one) and the ordered combine
// in one launch.  Workgroup u owns output rows 32u .. 32u+31 (tile u%4 of
// strip u/4 of every down plane) for all kk slots, so the combine needs no
// other workgroup's results.  Wavefront w takes k-steps w, w+8, ... of every
// slot, as the gathered down launch does, and requests the pieces of all kk
// slots before it waits for any: one memory round trip per 8 k-steps for the
// whole token.  The per-slot sums meet in LDS in wavefront order (the order,
// and so the bits, of the gathered down launch and its partials), and lanes
// 0..31 of wavefront 0 then run the combine's chain over the slots (the
// chain of combine_kernel).  The partials are written as well.
constexpr int DC_SB = DECODE_FUSED_MAX_SLOTS;  // slots per token this launch serves
struct Piece1 {
  v4u w[KSTEP];  // codes of blocks 0..3 (lane: row l%32, half l/32 of each block)
  v2u s[2];      // scale pair words of blocks 0-1 and 2-3
};

__device__ __forceinline__ void compute_piece1(const Piece1& p, const int8_t* act, const uint16_t* as, int lane,
                                               float& acc) {
  const float sw[KSTEP] = {h2f(p.s[0][0]), h2f(p.s[0][1]), h2f(p.s[1][0]), h2f(p.s[1][1])};
  const int8_t* arow = act + (lane >> 5) * 16;
  uint4 av[KSTEP];
#pragma unroll
  for (int kbi = 0; kbi < KSTEP; ++kbi) av[kbi] = *reinterpret_cast<const uint4*>(arow + kbi * 32);
  const uint2 s2 = *reinterpret_cast<const uint2*>(as);
  const float sa[KSTEP] = {h2f(s2.x), h2f(s2.x >> 16), h2f(s2.y), h2f(s2.y >> 16)};
#pragma unroll
  for (int kbi = 0; kbi < KSTEP; ++kbi) {
    const v4u wv = p.w[kbi];
    int dot = __builtin_amdgcn_sdot4((int)wv[0], (int)av[kbi].x, 0, false);
    dot = __builtin_amdgcn_sdot4((int)wv[1], (int)av[kbi].y, dot, false);
    dot = __builtin_amdgcn_sdot4((int)wv[2], (int)av[kbi].z, dot, false);
    dot = __builtin_amdgcn_sdot4((int)wv[3], (int)av[kbi].w, dot, false);
    acc = __builtin_fmaf((float)dot, sw[kbi] * sa[kbi], acc);
  }
}

__global__ __launch_bounds__(DW * 64) void decode_down_combine_kernel(DecodeArgs a, const float* __restrict__ gs,
                                                                      float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) int8_t s_act[DC_SB][DW * 128];      // the pass's h codes per slot
  __shared__ __attribute__((aligned(16))) uint16_t s_as[DC_SB][DW * KSTEP];   // and their scales
  __shared__ float red[DW][DC_SB][32];
  __shared__ float ys[DC_SB][32];
  __shared__ int s_g[DC_SB], s_ks[DC_SB], s_ex[DC_SB];
  __shared__ float s_w[DC_SB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kk = a.kk, k = a.k, E = a.E;
  // slot s: expert ids[s] (s < k) or the shared expert, its k-step count,
  // scale exponent and combine weight
  if (tid < kk) {
    int g = tid < k ? a.ids[tid] : E;
    g = (g >= 0 && g <= E) ? g : 0;
    s_g[tid] = g;
    s_ks[tid] = ((g == E) ? a.Fs_pad : a.F_pad) / (KSTEP * QB);
    s_w[tid] = tid < k ? a.w[tid] : gs[0];
  }
  __syncthreads();
  // the slots' scale exponents are needed only at the end: requested after
  // the first pass's pieces, so that no round trip precedes the weights
  int exv = 0;
  const int KSM = a.kmax_pad / (KSTEP * QB);
  const int strip = blockIdx.x >> 2, tsel = blockIdx.x & 3;
  const uint32_t o_code = (uint32_t)lane * 16, o_scale = (uint32_t)(lane & 31) * 8;
  float acc[DC_SB];
#pragma unroll
  for (int i = 0; i < DC_SB; ++i) acc[i] = 0.0f;

  for (int ks0 = 0; ks0 < KSM; ks0 += DW) {
    const int kq = ks0 + wave;  // this wavefront's k-step of the pass
    // the pass's h rows (slot s: pair row s), requested first: thread q moves
    // 16-byte piece q and q + 512 of the DC_SB x 64, thread q < DC_SB * DW the
    // 4 scales of (slot q / DW, k-step q % DW); pieces past a slot's k-steps
    // are not moved (and not read)
    uint4 hv[2];
    bool hok[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int q = tid + h * DW * 64, i = q >> 6, j = (q >> 3) & 7, c16 = q & 7;
      const int ic = min(i, kk - 1);
      hok[h] = i < kk && ks0 + j < s_ks[ic];
      hv[h] = hok[h] ? *reinterpret_cast<const uint4*>(a.hq + (size_t)ic * a.kmax_pad + (ks0 + j) * 128 + c16 * 16)
                     : make_uint4(0u, 0u, 0u, 0u);
    }
    const int si = min(tid / DW, kk - 1), sj = tid % DW;
    const bool sok = tid < DC_SB * DW && tid / DW < kk && ks0 + sj < s_ks[si];
    const uint2 sv = sok ? reinterpret_cast<const uint2*>(a.hs + (size_t)si * (a.kmax_pad / QB))[ks0 + sj]
                         : make_uint2(0u, 0u);
    // the pieces of every slot (a k-step past a slot's last re-reads its last
    // one and is not computed)
    Piece1 p[DC_SB];
#pragma unroll
    for (int i = 0; i < DC_SB; ++i) {
      const int s = min(i, kk - 1);
      const int g = __builtin_amdgcn_readfirstlane(s_g[s]);
      const int KSs = __builtin_amdgcn_readfirstlane(s_ks[s]);
      const uint8_t* plane = (g == E ? a.sh_dn : a.dn + (size_t)g * a.dn_group) + (size_t)strip * KSs * DN_KSTEP_BYTES;
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(plane), (short)0, -1, BUF_DWORD3);
      const int step_off = min(kq, KSs - 1) * DN_KSTEP_BYTES;
#pragma unroll
      for (int kbi = 0; kbi < KSTEP; ++kbi)
        p[i].w[kbi] = __builtin_amdgcn_raw_buffer_load_b128(rs, o_code, step_off + (kbi * 4 + tsel) * 1024, 0);
#pragma unroll
      for (int h = 0; h < 2; ++h)
        p[i].s[h] = __builtin_amdgcn_raw_buffer_load_b64(rs, o_scale, step_off + 16 * 1024 + tsel * 512 + h * 256, 0);
    }
    if (ks0 == 0 && tid < kk) exv = a.dn_exp[s_g[tid]];
    __builtin_amdgcn_sched_barrier(0);  // every request is out before any wait
    lds_barrier();  // every wavefront is done with the previous pass's LDS
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int q = tid + h * DW * 64, i = q >> 6, r = q & 63;
      if (hok[h]) reinterpret_cast<uint4*>(s_act[i])[r] = hv[h];
    }
    if (sok) reinterpret_cast<uint2*>(s_as[si])[sj] = sv;
    lds_barrier();
#pragma unroll
    for (int i = 0; i < DC_SB; ++i)
      if (i < kk && kq < s_ks[i])
        compute_piece1(p[i], s_act[i] + (kq - ks0) * 128, s_as[i] + (kq - ks0) * KSTEP, lane, acc[i]);
  }

  // the lane pair (two halves of each block), then the wavefronts in order
#pragma unroll
  for (int i = 0; i < DC_SB; ++i) {
    const float v = acc[i] + __shfl_xor(acc[i], 32, 64);
    if (i < kk && lane < 32) red[wave][i][lane] = v;
  }
  if (tid < kk) s_ex[tid] = exv;
  __syncthreads();
  const int row0 = 32 * (int)blockIdx.x;
  if (tid < DC_SB * 32) {
    const int i = tid >> 5, r = tid & 31;
    if (i < kk) {
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < DW; ++w) v += red[w][i][r];
      v = ldexpf(v, s_ex[i] - 23);
      ys[i][r] = v;
      if (row0 + r < a.d) a.partial[(size_t)i * a.d + row0 + r] = v;
    }
  }
  __syncthreads();
  if (tid < 32 && row0 + tid < a.d) {
    float o = 0.0f;
    for (int s = 0; s < k; ++s) o = __builtin_fmaf(s_w[s], ys[s][tid], o);
    if (a.has_shared) o = __builtin_fmaf(s_w[k], ys[k][tid], o);
    out[row0 + tid] = o;
  }
}

}  // namespace

// Workgroups per CU that fit at once (registers and LDS), from the runtime's
// occupancy calculator: a grid of n_cu times this many has every workgroup
// resident from the start.
template <bool GATEUP>
int resident_per_cu() {
  static int cached = 0;
  if (cached == 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_gemv_kernel<GATEUP>, DW * 64, 0) != hipSuccess) {
      (void)hipGetLastError();
      nb = 1;
    }
    cached = std::max(nb, 1);
  }
  return cached;
}

hipError_t launch_decode_gateup(const DecodeArgs& a, hipStream_t s) {
  const long units = (long)a.n_bound * (a.kmax_pad / 32);
  const long grid = std::min<long>(units, (long)a.n_cu * resident_per_cu<true>());
  decode_gemv_kernel<true><<<(unsigned)grid, DW * 64, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_decode_down_combine(const DecodeArgs& a, const float* gs, float* out, hipStream_t s) {
  if (a.n != 1 || a.kk > DC_SB) return hipErrorInvalidValue;
  decode_down_combine_kernel<<<(unsigned)(a.d_pad / 32), DW * 64, 0, s>>>(a, gs, out);
  return hipGetLastError();
}

hipError_t launch_decode_down(const DecodeArgs& a, hipStream_t s) {
  const long units = (long)a.n_bound * (a.d_pad / 64);
  const long grid = std::min<long>(units, (long)a.n_cu * resident_per_cu<false>());
  decode_gemv_kernel<false><<<(unsigned)grid, DW * 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
