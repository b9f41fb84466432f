// api.hip -- host side of libmoe_ffn: argument validation, the weights handle,
// workspace carving and the launch sequence of one MoE FFN layer.
//
// One prefill call enqueues, on the caller's stream and without any host
// synchronisation or device-to-host transfer (the routing result stays on
// the device; SharpInference #388, "Remaining levers" 1):
//   1. router                   (fp32 fused-chain logits for all experts)
//   2. routing                  (top-k, softmax weights, per-tile expert
//                                histograms and ranks; in the router's
//                                launch when E <= 64)
//   3. bucketing                (CSR expStart/expTokI/expTokK, the 128-row tile
//                                table, each pair's padded GEMM row), then the
//                                int8 quantiser of x (and the shared-expert
//                                gate), which writes each token's codes to its
//                                expert slots' rows in GEMM operand form
//   4. grouped gate/up + SwiGLU (one launch over all experts + shared expert)
//   5. grouped down             (one launch; unweighted partials per slot)
//   6. ordered combine          (#129 "Scope")
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>

#include "internal.h"

using namespace moe;

namespace moe {

WsLayout ws_layout(const Dims& dm, int max_tokens) {
  WsLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  };
  const size_t Nn = (size_t)std::max(max_tokens, 1);
  const size_t kk = (size_t)dm.k + dm.has_shared;
  const size_t P_total = Nn * dm.k + (dm.has_shared ? Nn : 0);
  L.n_route_tiles = (int)((Nn + ROUTE_TILE - 1) / ROUTE_TILE);
  L.tile_bound = (int)((P_total + (size_t)(MT_WG - 1) * dm.G) / MT_WG + 1);
  const size_t kbmax = (size_t)dm.kmax_pad / QB;
  L.logits = take(Nn * dm.E * 4);
  L.ids = take(Nn * dm.k * 4);
  L.rank = take(Nn * dm.k * 4);
  L.w = take(Nn * dm.k * 4);
  L.gs = take(Nn * 4);
  L.hist = take((size_t)L.n_route_tiles * dm.E * 4);
  L.exp_start = take((size_t)(dm.E + 2) * 4);
  L.tok_i = take(P_total * 4);
  L.tok_k = take(P_total * 4);
  L.row_tok = take((size_t)L.tile_bound * MT_WG * 4);
  L.tiles = take((4 + 3 * (size_t)L.tile_bound) * 4);
  const size_t t32 = (size_t)L.tile_bound * (MT_WG / MT_WAVE);
  const size_t kbd = (size_t)dm.d_pad / QB;
  L.gq = take(Nn * dm.d_pad);        // token-major codes
  L.gxs = take(dm.E > 64 ? Nn * kbd * 2 : 0);  // and their scales, when the routing launch quantises
  L.gqs = take(t32 * 32 * kbd * 2);  // their scales per tile row
  L.hq = take(t32 * kbmax * 1024);
  L.hs = take(t32 * 32 * kbmax * 2);
  L.partial = take(Nn * kk * dm.d * 4);
  // The decode region is always reserved, for min(max_tokens, 8) tokens, so
  // that the total never shrinks as max_tokens grows: a workspace sized once
  // for max_tokens serves every call with fewer tokens, decode included.
  const size_t Nd = std::min(Nn, (size_t)DECODE_MAX_TOKENS);
  const size_t nb = std::min((size_t)dm.E, Nd * dm.k) + dm.has_shared;
  L.dlist = take((4 + DLIST_ENTRY * nb) * 4);
  L.dxq = take(Nd * dm.d_pad);
  L.dxs = take(Nd * (dm.d_pad / QB) * 2);
  L.dhq = take(Nd * kk * dm.kmax_pad);
  L.dhs = take(Nd * kk * (dm.kmax_pad / QB) * 2);
  L.total = off;
  return L;
}

}  // namespace moe

namespace {

constexpr int MAX_TOKENS = 1 << 20;

int check_dims(const moe_ffn_dims* u) {
  if (!u) return MOE_FFN_INVALID_ARG;
  if (u->d_model <= 0 || u->d_ffn <= 0 || u->d_shared_ffn < 0 || u->n_experts <= 0 || u->top_k <= 0)
    return MOE_FFN_INVALID_ARG;
  if (u->norm_topk_prob != 0 && u->norm_topk_prob != 1) return MOE_FFN_INVALID_ARG;
  if (u->top_k > u->n_experts) return MOE_FFN_INVALID_ARG;
  if (u->d_model % QB || u->d_ffn % QB || u->d_shared_ffn % QB) return MOE_FFN_UNSUPPORTED;
  if (u->n_experts > MAX_EXPERTS || u->top_k > MAX_TOPK) return MOE_FFN_UNSUPPORTED;
  if (u->d_model > (1 << 16) || u->d_ffn > (1 << 16) || u->d_shared_ffn > (1 << 16))
    return MOE_FFN_UNSUPPORTED;
  return MOE_FFN_OK;
}

Dims make_dims(const moe_ffn_dims* u) {
  Dims dm{};
  dm.d = u->d_model;
  dm.E = u->n_experts;
  dm.k = u->top_k;
  dm.F = u->d_ffn;
  dm.Fs = u->d_shared_ffn;
  dm.norm = u->norm_topk_prob;
  dm.has_shared = u->d_shared_ffn > 0 ? 1 : 0;
  dm.d_pad = round_up(dm.d, KPAD);
  dm.F_pad = round_up(dm.F, KPAD);
  dm.Fs_pad = dm.has_shared ? round_up(dm.Fs, KPAD) : 0;
  dm.kmax_pad = std::max(dm.F_pad, dm.Fs_pad);
  dm.E64 = round_up(dm.E, 64);
  dm.G = dm.E + dm.has_shared;
  return dm;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
  return na && nb && pa < pb + nb && pb < pa + na;
}

#define HIP_TRY(expr)                                   \
  do {                                                  \
    if ((expr) != hipSuccess) return MOE_FFN_HIP_ERROR; \
  } while (0)

int current_device_matches(const moe_ffn_weights* w) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_FFN_HIP_ERROR;
  return dev == w->device ? MOE_FFN_OK : MOE_FFN_INVALID_ARG;
}

// The optional routing outputs of a call (device-to-device copies on s).
hipError_t copy_routing(const Dims& dm, int n, const moe_ffn_routing* r, const int32_t* ids,
                        const float* w, const float* gs, const int32_t* exp_start,
                        const int32_t* tok_i, const int32_t* tok_k, const float* partial,
                        hipStream_t s) {
  if (!r) return hipSuccess;
  const int kk = dm.k + dm.has_shared;
  const size_t nk = (size_t)n * dm.k;
  const size_t ptot = nk + (dm.has_shared ? (size_t)n : 0);
  hipError_t e = hipSuccess;
  auto cp = [&](void* dst, const void* src, size_t bytes) {
    if (e == hipSuccess && dst) e = hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s);
  };
  cp(r->topk_ids, ids, nk * 4);
  cp(r->topk_w, w, nk * 4);
  if (dm.has_shared) cp(r->shared_gate, gs, (size_t)n * 4);
  cp(r->exp_start, exp_start, (size_t)(dm.E + 1 + dm.has_shared) * 4);
  cp(r->exp_tok_i, tok_i, ptot * 4);
  cp(r->exp_tok_k, tok_k, ptot * 4);
  cp(r->partial, partial, (size_t)n * kk * dm.d * 4);
  return e;
}

// The arguments of the two grouped GEMMs of a call over n tokens whose
// workspace (laid out as L) starts at base.
GemmArgs gemm_args(const moe_ffn_weights* W, const WsLayout& L, char* base, int n) {
  const Dims& dm = W->dm;
  GemmArgs a{};
  a.tiles = (const int32_t*)(base + L.tiles);
  a.tok_i = (const int32_t*)(base + L.tok_i);
  a.tok_k = (const int32_t*)(base + L.tok_k);
  a.row_tok = (const int32_t*)(base + L.row_tok);
  a.E = dm.E;
  a.G = dm.G;
  a.n_tokens = n;
  a.p_total = n * dm.k + (dm.has_shared ? n : 0);
  a.tile_bound = L.tile_bound;
  a.kbmax = dm.kmax_pad / QB;
  a.hq = (int8_t*)(base + L.hq);
  a.hs = (uint16_t*)(base + L.hs);
  a.gq = (const int8_t*)(base + L.gq);
  a.gqs = (const uint16_t*)(base + L.gqs);
  a.d_pad = dm.d_pad;
  a.gu = W->gu;
  a.gu_group = W->gu_per_expert;
  a.sh_gu = W->sh_gu;
  a.F_pad = dm.F_pad;
  a.Fs_pad = dm.Fs_pad;
  a.dn = W->dn;
  a.dn_group = W->dn_per_expert;
  a.sh_dn = W->sh_dn;
  a.dn_exp = W->dn_exp;
  a.partial = (float*)(base + L.partial);
  a.d = dm.d;
  a.kk = dm.k + dm.has_shared;
  return a;
}

// The stack form of a layer: instead of writing the layer's output, its
// combine adds it to the residual stream h and writes the next layer's
// input xn = RMSNorm(h).
struct ResidualOut {
  float* h;
  float* xn;
  float eps;
};

int run_layer(const moe_ffn_weights* W, const float* x, int32_t n, float* out, void* ws,
              size_t ws_bytes, const moe_ffn_routing* r, hipStream_t s, hipEvent_t* ev = nullptr,
              const ResidualOut* res = nullptr, int reverse_tiles = 0) {
  if (!W || n < 0 || n > MAX_TOKENS) return MOE_FFN_INVALID_ARG;
  // gate/up addresses its token-major activation codes by 32-bit offsets
  if ((uint64_t)n * (uint64_t)W->dm.d_pad > 0xffffff00ull) return MOE_FFN_INVALID_ARG;
  if (n == 0) return current_device_matches(W);  // no-op; buffers may be NULL
  if (!x || !ws || (!res && !out)) return MOE_FFN_INVALID_ARG;
  const Dims& dm = W->dm;
  const WsLayout L = ws_layout(dm, n);
  if (ws_bytes < L.total) return MOE_FFN_WORKSPACE_TOO_SMALL;
  if (((uintptr_t)ws & 255u) || ((uintptr_t)x & 15u) || (!res && ((uintptr_t)out & 15u)))
    return MOE_FFN_INVALID_ARG;
  const size_t xb = (size_t)n * dm.d * sizeof(float);
  if (res) {
    // xn may be x itself: x is last read before the combine runs
    if (!res->h || !res->xn || !(res->eps >= 0.0f)) return MOE_FFN_INVALID_ARG;
    if (((uintptr_t)res->h & 15u) || ((uintptr_t)res->xn & 15u)) return MOE_FFN_INVALID_ARG;
    if (overlaps(res->h, xb, x, xb) || overlaps(res->h, xb, ws, ws_bytes) ||
        overlaps(res->xn, xb, res->h, xb) || overlaps(res->xn, xb, ws, ws_bytes) ||
        (res->xn != x && overlaps(res->xn, xb, x, xb)))
      return MOE_FFN_INVALID_ARG;
  } else if (overlaps(x, xb, out, xb) || overlaps(out, xb, ws, ws_bytes)) {
    return MOE_FFN_INVALID_ARG;
  }
  if (r && r->xq && ((uintptr_t)r->xq & 15u)) return MOE_FFN_INVALID_ARG;
  const int dev_ok = current_device_matches(W);
  if (dev_ok != MOE_FFN_OK) return dev_ok;

  char* base = (char*)ws;
  float* logits = (float*)(base + L.logits);
  int32_t* ids = (int32_t*)(base + L.ids);
  int32_t* rank = (int32_t*)(base + L.rank);
  float* w = (float*)(base + L.w);
  float* gs = (float*)(base + L.gs);
  int32_t* hist = (int32_t*)(base + L.hist);
  int32_t* exp_start = (int32_t*)(base + L.exp_start);
  int32_t* tok_i = (int32_t*)(base + L.tok_i);
  int32_t* tok_k = (int32_t*)(base + L.tok_k);
  int32_t* tiles = (int32_t*)(base + L.tiles);
  int8_t* gq = (int8_t*)(base + L.gq);
  uint16_t* gqs = (uint16_t*)(base + L.gqs);
  float* partial = (float*)(base + L.partial);
  const int kk = dm.k + dm.has_shared;
  auto mark = [&](int i) { return ev ? hipEventRecord(ev[i], s) : hipSuccess; };

  HIP_TRY(mark(0));
  const float* rbias = W->has_bias ? W->router_bias : nullptr;
  if (dm.E <= 64) {
    // one workgroup holds all logits of its tokens: router and routing fused
    HIP_TRY(launch_router_route(x, n, dm.d, W->router_wt, rbias, dm.E, dm.k, dm.norm, ids, w, rank,
                                hist, W->n_cu, s));
    HIP_TRY(mark(1));
  } else {
    HIP_TRY(launch_router(x, n, dm.d, W->router_wt, rbias, dm.E, dm.E64, logits, W->n_cu, s));
    HIP_TRY(mark(1));
    // the routing launch also quantises the tokens (its routing workgroups fill few CUs)
    const RowQuant rq{x, dm.d, dm.d_pad, dm.has_shared ? W->sh_gate_vec : nullptr, gs, gq,
                      (uint16_t*)(base + L.gxs), r ? r->xq : nullptr, r ? r->xs : nullptr};
    HIP_TRY(launch_route(logits, n, dm.E, dm.k, dm.norm, ids, w, rank, hist, rq, s));
  }
  HIP_TRY(mark(2));
  const bool quantised = dm.E > 64;
  HIP_TRY(launch_bucket_quantize(ids, rank, hist, n, dm.E, dm.k, dm.has_shared, exp_start, tok_i, tok_k,
                                 (int32_t*)(base + L.row_tok),
                                 tiles, L.tile_bound, x, dm.d, dm.d_pad, gq, gqs,
                                 dm.has_shared ? W->sh_gate_vec : nullptr, gs,
                                 (r && !quantised) ? r->xq : nullptr, (r && !quantised) ? r->xs : nullptr,
                                 quantised ? (const uint16_t*)(base + L.gxs) : nullptr, s));
  GemmArgs a = gemm_args(W, L, base, n);
  a.reverse = reverse_tiles;
  HIP_TRY(mark(3));
  const bool q4k = W->fmt == MOE_FFN_FMT_Q4_K;
  HIP_TRY(q4k ? launch_gateup_q4k(a, s) : launch_gateup(a, s));
  HIP_TRY(mark(4));
  HIP_TRY(q4k ? launch_down_q4k(a, s) : launch_down(a, s));
  HIP_TRY(mark(5));
  if (res)
    HIP_TRY(launch_combine_residual_rmsnorm(partial, w, dm.has_shared ? gs : nullptr, n, dm.k, kk, dm.d,
                                            res->h, res->xn, res->eps, s));
  else
    HIP_TRY(launch_combine(partial, w, dm.has_shared ? gs : nullptr, n, dm.k, kk, dm.d, out, s));
  HIP_TRY(mark(6));

  HIP_TRY(copy_routing(dm, n, r, ids, w, gs, exp_start, tok_i, tok_k, partial, s));
  return MOE_FFN_OK;
}


// Decode (1 <= n <= DECODE_MAX_TOKENS): router chains spread over the chip
// (plus the token-major quantiser), the gate/up matvec launch (which also
// routes the tokens and lists the active groups), the down matvec launch over
// that list, and the ordered combine (#408 "Hypothesis" levers 1 and 3).
int run_decode(const moe_ffn_weights* W, const float* x, int32_t n, float* out, void* ws,
               size_t ws_bytes, const moe_ffn_routing* r, hipStream_t s, hipEvent_t* ev = nullptr) {
  if (!W || n < 1 || n > DECODE_MAX_TOKENS) return MOE_FFN_INVALID_ARG;
  if (!x || !out || !ws) return MOE_FFN_INVALID_ARG;
  // The gathered matvecs read the Q8_0 planes; Q4_K planes go through the
  // prefill launches.  The decode stage events then bracket router, routing
  // and bucketing + quantiser (event 1 is recorded again before each of
  // those launches' successors, and its last record counts), gate/up, down
  // and the combine.
  if (W->fmt != MOE_FFN_FMT_Q8_0) {
    if (!ev) return run_layer(W, x, n, out, ws, ws_bytes, r, s);
    hipEvent_t pe[MOE_FFN_N_STAGE_EVENTS] = {ev[0], ev[1], ev[1], ev[1], ev[2], ev[3], ev[4]};
    return run_layer(W, x, n, out, ws, ws_bytes, r, s, pe);
  }
  const Dims& dm = W->dm;
  const WsLayout L = ws_layout(dm, n);
  if (ws_bytes < L.total) return MOE_FFN_WORKSPACE_TOO_SMALL;
  if (((uintptr_t)ws & 255u) || ((uintptr_t)x & 15u) || ((uintptr_t)out & 15u))
    return MOE_FFN_INVALID_ARG;
  const size_t xb = (size_t)n * dm.d * sizeof(float);
  if (overlaps(x, xb, out, xb) || overlaps(out, xb, ws, ws_bytes)) return MOE_FFN_INVALID_ARG;
  if (r && r->xq && ((uintptr_t)r->xq & 15u)) return MOE_FFN_INVALID_ARG;
  const int dev_ok = current_device_matches(W);
  if (dev_ok != MOE_FFN_OK) return dev_ok;

  char* base = (char*)ws;
  float* logits = (float*)(base + L.logits);
  int32_t* ids = (int32_t*)(base + L.ids);
  float* w = (float*)(base + L.w);
  float* gs = (float*)(base + L.gs);
  int32_t* exp_start = (int32_t*)(base + L.exp_start);
  int32_t* tok_i = (int32_t*)(base + L.tok_i);
  int32_t* tok_k = (int32_t*)(base + L.tok_k);
  int32_t* dlist = (int32_t*)(base + L.dlist);
  int8_t* dxq = (int8_t*)(base + L.dxq);
  uint16_t* dxs = (uint16_t*)(base + L.dxs);
  float* partial = (float*)(base + L.partial);
  const int kk = dm.k + dm.has_shared;
  auto mark = [&](int i) { return ev ? hipEventRecord(ev[i], s) : hipSuccess; };

  HIP_TRY(mark(0));
  HIP_TRY(launch_decode_router(x, n, dm.d, dm.d_pad, W->router_wt, W->has_bias ? W->router_bias : nullptr,
                               dm.E, dm.E64, logits, dm.has_shared ? W->sh_gate_vec : nullptr, gs, dxq,
                               dxs, s));
  HIP_TRY(mark(1));
  DecodeArgs a{};
  a.logits = logits;
  a.n = n;
  a.k = dm.k;
  a.norm = dm.norm;
  a.has_shared = dm.has_shared;
  a.ids = ids;
  a.w = w;
  a.exp_start = exp_start;
  a.tok_i = tok_i;
  a.tok_k = tok_k;
  a.dlist = dlist;
  a.E = dm.E;
  a.kk = kk;
  a.n_bound = std::min(dm.E, n * dm.k) + dm.has_shared;
  a.n_cu = W->n_cu;
  a.xq = dxq;
  a.xs = dxs;
  a.gu = W->gu;
  a.gu_group = W->gu_per_expert;
  a.sh_gu = W->sh_gu;
  a.d = dm.d;
  a.d_pad = dm.d_pad;
  a.F_pad = dm.F_pad;
  a.Fs_pad = dm.Fs_pad;
  a.kmax_pad = dm.kmax_pad;
  a.hq = (int8_t*)(base + L.dhq);
  a.hs = (uint16_t*)(base + L.dhs);
  a.dn = W->dn;
  a.dn_group = W->dn_per_expert;
  a.sh_dn = W->sh_dn;
  a.dn_exp = W->dn_exp;
  a.partial = partial;
  HIP_TRY(launch_decode_gateup(a, s));
  HIP_TRY(mark(2));
  if (n == 1 && kk <= DECODE_FUSED_MAX_SLOTS) {
    // one token: down matvec and combine in one launch (stage 3 is empty)
    HIP_TRY(launch_decode_down_combine(a, gs, out, s));
    HIP_TRY(mark(3));
  } else {
    HIP_TRY(launch_decode_down(a, s));
    HIP_TRY(mark(3));
    HIP_TRY(launch_combine(partial, w, dm.has_shared ? gs : nullptr, n, dm.k, kk, dm.d, out, s));
  }
  HIP_TRY(mark(4));

  HIP_TRY(copy_routing(dm, n, r, ids, w, gs, exp_start, tok_i, tok_k, partial, s));
  if (r && r->xq)
    HIP_TRY(hipMemcpy2DAsync(r->xq, (size_t)dm.d, dxq, (size_t)dm.d_pad, (size_t)dm.d, (size_t)n,
                             hipMemcpyDeviceToDevice, s));
  if (r && r->xs)
    HIP_TRY(hipMemcpy2DAsync(r->xs, (size_t)(dm.d / QB) * 2, dxs, (size_t)(dm.d_pad / QB) * 2,
                             (size_t)(dm.d / QB) * 2, (size_t)n, hipMemcpyDeviceToDevice, s));
  return MOE_FFN_OK;
}

}  // namespace

extern "C" {

int moe_ffn_weights_create(const moe_ffn_dims* dims, const float* router_w,
                           const float* router_bias, const void* gate_q8, const void* up_q8,
                           const void* down_q8, const void* sh_gate_q8, const void* sh_up_q8,
                           const void* sh_down_q8, const float* sh_gate_vec, hipStream_t stream,
                           moe_ffn_weights** out) {
  return moe_ffn_weights_create_fmt(dims, MOE_FFN_FMT_Q8_0, router_w, router_bias, gate_q8, up_q8, down_q8,
                                    sh_gate_q8, sh_up_q8, sh_down_q8, sh_gate_vec, stream, out);
}

int moe_ffn_weights_create_fmt(const moe_ffn_dims* dims, int32_t format, const float* router_w,
                               const float* router_bias, const void* gate, const void* up,
                               const void* down, const void* sh_gate, const void* sh_up,
                               const void* sh_down, const float* sh_gate_vec, hipStream_t stream,
                               moe_ffn_weights** out) {
  if (!out) return MOE_FFN_INVALID_ARG;
  *out = nullptr;
  if (format != MOE_FFN_FMT_Q8_0 && format != MOE_FFN_FMT_Q4_K && format != MOE_FFN_FMT_Q3_K)
    return MOE_FFN_INVALID_ARG;
  const int rc = check_dims(dims);
  if (rc != MOE_FFN_OK) return rc;
  const bool q4k = format == MOE_FFN_FMT_Q4_K;
  if (format != MOE_FFN_FMT_Q8_0 &&
      (dims->d_model % Q4K_VALUES || dims->d_ffn % Q4K_VALUES || dims->d_shared_ffn % Q4K_VALUES))
    return MOE_FFN_UNSUPPORTED;
  if (!router_w || !gate || !up || !down) return MOE_FFN_INVALID_ARG;
  const bool has_sh = dims->d_shared_ffn > 0;
  const bool any_sh = sh_gate || sh_up || sh_down || sh_gate_vec;
  const bool all_sh = sh_gate && sh_up && sh_down && sh_gate_vec;
  if (has_sh ? !all_sh : any_sh) return MOE_FFN_INVALID_ARG;

  moe_ffn_weights* W = new (std::nothrow) moe_ffn_weights();
  if (!W) return MOE_FFN_OUT_OF_MEMORY;
  W->user = *dims;
  W->dm = make_dims(dims);
  W->fmt = format == MOE_FFN_FMT_Q3_K ? MOE_FFN_FMT_Q8_0 : format;  // Q3_K runs on Q8_0 planes
  const Dims& dm = W->dm;
  if (hipGetDevice(&W->device) != hipSuccess ||
      hipDeviceGetAttribute(&W->n_cu, hipDeviceAttributeMultiprocessorCount, W->device) != hipSuccess ||
      W->n_cu <= 0) {
    (void)hipGetLastError();
    delete W;
    return MOE_FFN_HIP_ERROR;
  }
  W->has_bias = router_bias ? 1 : 0;
  // [strips][k-steps][k-step bytes] per expert (see internal.h)
  const size_t gu_step = q4k ? Q4K_KSTEP_BYTES : KSTEP_BYTES;
  const size_t dn_step = q4k ? Q4K_KSTEP_BYTES : DN_KSTEP_BYTES;
  W->gu_per_expert = (size_t)(dm.F_pad / GU_COLS) * (dm.d_pad / QB / KSTEP) * gu_step;
  W->dn_per_expert = (size_t)(dm.d_pad / DN_COLS) * (dm.F_pad / QB / KSTEP) * dn_step;
  const size_t sh_gu = (size_t)(dm.Fs_pad / GU_COLS) * (dm.d_pad / QB / KSTEP) * gu_step;
  const size_t sh_dn = (size_t)(dm.d_pad / DN_COLS) * (dm.Fs_pad / QB / KSTEP) * dn_step;

  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  };
  const size_t o_rw = take((size_t)dm.d * dm.E64 * 4);
  const size_t o_rb = take((size_t)dm.E * 4);
  const size_t o_sg = take((size_t)dm.d * 4);
  const size_t o_ex = take((size_t)dm.G * 4);
  const size_t o_of = take(4);  // Q4_K repack overflow flag
  const size_t o_gu = take(W->gu_per_expert * dm.E);
  const size_t o_dn = take(W->dn_per_expert * dm.E);
  const size_t o_sgu = take(sh_gu), o_sdn = take(sh_dn);
  if (hipMalloc(&W->base, off) != hipSuccess) {
    (void)hipGetLastError();
    delete W;
    return MOE_FFN_OUT_OF_MEMORY;
  }
  char* b = (char*)W->base;
  W->router_wt = (float*)(b + o_rw);
  W->router_bias = (float*)(b + o_rb);
  W->sh_gate_vec = (float*)(b + o_sg);
  W->dn_exp = (int32_t*)(b + o_ex);
  int32_t* overflow = (int32_t*)(b + o_of);
  W->gu = (uint8_t*)(b + o_gu);
  W->dn = (uint8_t*)(b + o_dn);
  W->sh_gu = has_sh ? (uint8_t*)(b + o_sgu) : nullptr;
  W->sh_dn = has_sh ? (uint8_t*)(b + o_sdn) : nullptr;

  hipError_t e = hipSuccess;
  void* tmp = nullptr;  // Q3_K: the expanded Q8_0 rows (load time only)
  if (e == hipSuccess) e = launch_transpose_router(router_w, dm.E, dm.d, dm.E64, W->router_wt, stream);
  if (e == hipSuccess)
    e = router_bias ? hipMemcpyAsync(W->router_bias, router_bias, (size_t)dm.E * 4, hipMemcpyDeviceToDevice, stream)
                    : hipMemsetAsync(W->router_bias, 0, (size_t)dm.E * 4, stream);
  if (e == hipSuccess)
    e = has_sh ? hipMemcpyAsync(W->sh_gate_vec, sh_gate_vec, (size_t)dm.d * 4, hipMemcpyDeviceToDevice, stream)
               : hipMemsetAsync(W->sh_gate_vec, 0, (size_t)dm.d * 4, stream);
  if (q4k) {
    // the down planes carry no rescaling exponent (the epilogue's 2^e is 1)
    const int nsd = dm.d / Q4K_VALUES, nsf = dm.F / Q4K_VALUES;
    const size_t row_d = (size_t)nsd * Q4K_BYTES, row_f = (size_t)nsf * Q4K_BYTES;
    if (e == hipSuccess) e = hipMemsetAsync(W->dn_exp, 0, (size_t)dm.G * 4, stream);
    if (e == hipSuccess) e = hipMemsetAsync(overflow, 0, 4, stream);
    if (e == hipSuccess)
      e = launch_repack_q4k((const uint8_t*)gate, (const uint8_t*)up, dm.E, (size_t)dm.F * row_d, dm.F, nsd, 2,
                            dm.F_pad / GU_COLS, dm.d_pad / QB / KSTEP, W->gu, W->gu_per_expert, overflow, stream);
    if (e == hipSuccess)
      e = launch_repack_q4k((const uint8_t*)down, (const uint8_t*)down, dm.E, (size_t)dm.d * row_f, dm.d, nsf, 4,
                            dm.d_pad / DN_COLS, dm.F_pad / QB / KSTEP, W->dn, W->dn_per_expert, overflow, stream);
    if (e == hipSuccess && has_sh) {
      const int nss = dm.Fs / Q4K_VALUES;
      e = launch_repack_q4k((const uint8_t*)sh_gate, (const uint8_t*)sh_up, 1, (size_t)dm.Fs * row_d, dm.Fs, nsd,
                            2, dm.Fs_pad / GU_COLS, dm.d_pad / QB / KSTEP, W->sh_gu, sh_gu, overflow, stream);
      if (e == hipSuccess)
        e = launch_repack_q4k((const uint8_t*)sh_down, (const uint8_t*)sh_down, 1,
                              (size_t)dm.d * nss * Q4K_BYTES, dm.d, nss, 4, dm.d_pad / DN_COLS,
                              dm.Fs_pad / QB / KSTEP, W->sh_dn, sh_dn, overflow, stream);
    }
  } else {
    // Q8_0 rows: as given, or (Q3_K) expanded at load into Q8_0 rows with the
    // same values, all six matrices in one temporary buffer freed below
    const int nbd = dm.d / QB, nbf = dm.F / QB, nbs = dm.Fs / QB;
    const size_t q8_gu = (size_t)dm.F * nbd * Q8_BYTES, q8_dn = (size_t)dm.d * nbf * Q8_BYTES;
    const size_t q8_sgu = (size_t)dm.Fs * nbd * Q8_BYTES, q8_sdn = (size_t)dm.d * nbs * Q8_BYTES;
    const void *g8 = gate, *u8 = up, *d8 = down, *sg8 = sh_gate, *su8 = sh_up, *sd8 = sh_down;
    if (format == MOE_FFN_FMT_Q3_K && e == hipSuccess) {
      const size_t total = dm.E * (2 * q8_gu + q8_dn) + 2 * q8_sgu + q8_sdn;
      if (hipMalloc(&tmp, total) != hipSuccess) {
        (void)hipGetLastError();
        (void)hipFree(W->base);
        delete W;
        return MOE_FFN_OUT_OF_MEMORY;
      }
      {
        uint8_t* p = (uint8_t*)tmp;
        const int ssd = dm.d / Q4K_VALUES, ssf = dm.F / Q4K_VALUES, sss = dm.Fs / Q4K_VALUES;
        const size_t row_d = (size_t)ssd * Q3K_BYTES, row_f = (size_t)ssf * Q3K_BYTES;
        auto expand = [&](const void* src, int groups, size_t src_group, int rows, int supers, size_t dst_group,
                          const void** dst) {
          if (e == hipSuccess) e = launch_q3k_to_q8((const uint8_t*)src, groups, src_group, rows, supers, p, dst_group, stream);
          *dst = p;
          p += (size_t)groups * dst_group;
        };
        expand(gate, dm.E, (size_t)dm.F * row_d, dm.F, ssd, q8_gu, &g8);
        expand(up, dm.E, (size_t)dm.F * row_d, dm.F, ssd, q8_gu, &u8);
        expand(down, dm.E, (size_t)dm.d * row_f, dm.d, ssf, q8_dn, &d8);
        if (has_sh) {
          expand(sh_gate, 1, (size_t)dm.Fs * row_d, dm.Fs, ssd, q8_sgu, &sg8);
          expand(sh_up, 1, (size_t)dm.Fs * row_d, dm.Fs, ssd, q8_sgu, &su8);
          expand(sh_down, 1, (size_t)dm.d * sss * Q3K_BYTES, dm.d, sss, q8_sdn, &sd8);
        }
      }
    }
    if (e == hipSuccess)
      e = launch_repack_q8((const uint8_t*)g8, (const uint8_t*)u8, dm.E, q8_gu, dm.F, nbd, 2, dm.F_pad / GU_COLS,
                           dm.d_pad / QB, W->gu, W->gu_per_expert, nullptr, stream);
    if (e == hipSuccess)
      e = launch_scale_exponent((const uint8_t*)d8, dm.E, q8_dn, (long)dm.d * nbf, W->dn_exp, stream);
    if (e == hipSuccess)
      e = launch_repack_q8((const uint8_t*)d8, (const uint8_t*)d8, dm.E, q8_dn, dm.d, nbf, 4, dm.d_pad / DN_COLS,
                           dm.F_pad / QB, W->dn, W->dn_per_expert, W->dn_exp, stream);
    if (e == hipSuccess && has_sh) {
      e = launch_repack_q8((const uint8_t*)sg8, (const uint8_t*)su8, 1, q8_sgu, dm.Fs, nbd, 2, dm.Fs_pad / GU_COLS,
                           dm.d_pad / QB, W->sh_gu, sh_gu, nullptr, stream);
      if (e == hipSuccess)
        e = launch_scale_exponent((const uint8_t*)sd8, 1, q8_sdn, (long)dm.d * nbs, W->dn_exp + dm.E, stream);
      if (e == hipSuccess)
        e = launch_repack_q8((const uint8_t*)sd8, (const uint8_t*)sd8, 1, q8_sdn, dm.d, nbs, 4, dm.d_pad / DN_COLS,
                             dm.Fs_pad / QB, W->sh_dn, sh_dn, W->dn_exp + dm.E, stream);
    }
  }
  int32_t overflow_h = 0;
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (tmp && hipFree(tmp) != hipSuccess && e == hipSuccess) e = hipErrorUnknown;
  if (e == hipSuccess && q4k) e = hipMemcpy(&overflow_h, overflow, 4, hipMemcpyDeviceToHost);
  if (e != hipSuccess || overflow_h) {
    (void)hipGetLastError();
    (void)hipFree(W->base);
    delete W;
    return e != hipSuccess ? MOE_FFN_HIP_ERROR : MOE_FFN_UNSUPPORTED;
  }
  *out = W;
  return MOE_FFN_OK;
}

int moe_ffn_weights_destroy(moe_ffn_weights* w) {
  if (!w) return MOE_FFN_OK;
  const hipError_t e = hipFree(w->base);
  delete w;
  return e == hipSuccess ? MOE_FFN_OK : MOE_FFN_HIP_ERROR;
}

int moe_ffn_weights_dims(const moe_ffn_weights* w, moe_ffn_dims* dims_out) {
  if (!w || !dims_out) return MOE_FFN_INVALID_ARG;
  *dims_out = w->user;
  return MOE_FFN_OK;
}

int moe_ffn_workspace_size(const moe_ffn_weights* w, int32_t max_tokens, size_t* bytes) {
  if (!w || !bytes || max_tokens < 0 || max_tokens > MAX_TOKENS) return MOE_FFN_INVALID_ARG;
  *bytes = ws_layout(w->dm, max_tokens).total;
  return MOE_FFN_OK;
}

int moe_ffn_workspace_size_for_dims(const moe_ffn_dims* dims, int32_t max_tokens, size_t* bytes) {
  if (!bytes || max_tokens < 0 || max_tokens > MAX_TOKENS) return MOE_FFN_INVALID_ARG;
  const int rc = check_dims(dims);
  if (rc != MOE_FFN_OK) return rc;
  *bytes = ws_layout(make_dims(dims), max_tokens).total;
  return MOE_FFN_OK;
}

int moe_ffn_prefill(const moe_ffn_weights* w, const float* x, int32_t n_tokens, float* out,
                    void* ws, size_t ws_bytes, const moe_ffn_routing* routing, hipStream_t stream) {
  return run_layer(w, x, n_tokens, out, ws, ws_bytes, routing, stream);
}

int moe_ffn_prefill_chunked(const moe_ffn_weights* w, const float* x, int32_t n_tokens,
                            int32_t chunk_tokens, int32_t flags, float* out, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  if (!w || n_tokens < 0 || n_tokens > MAX_TOKENS || chunk_tokens < 1 || (flags & ~MOE_FFN_CHUNK_SERPENTINE))
    return MOE_FFN_INVALID_ARG;
  if (n_tokens == 0) return current_device_matches(w);
  if (!x || !out || !ws) return MOE_FFN_INVALID_ARG;
  // Every chunk's checks, done once before anything is enqueued: the
  // workspace covers the largest chunk, and the whole of x and out.
  const int32_t m0 = std::min(chunk_tokens, n_tokens);
  if (ws_bytes < ws_layout(w->dm, m0).total) return MOE_FFN_WORKSPACE_TOO_SMALL;
  if (((uintptr_t)ws & 255u) || ((uintptr_t)x & 15u) || ((uintptr_t)out & 15u)) return MOE_FFN_INVALID_ARG;
  const size_t xb = (size_t)n_tokens * w->dm.d * sizeof(float);
  if (overlaps(x, xb, out, xb) || overlaps(out, xb, ws, ws_bytes)) return MOE_FFN_INVALID_ARG;
  const int dev_ok = current_device_matches(w);
  if (dev_ok != MOE_FFN_OK) return dev_ok;
  for (int32_t c0 = 0, c = 0; c0 < n_tokens; c0 += chunk_tokens, ++c) {
    const int32_t m = std::min(chunk_tokens, n_tokens - c0);
    const size_t off = (size_t)c0 * w->dm.d;
    const int rev = (flags & MOE_FFN_CHUNK_SERPENTINE) ? (c & 1) : 0;
    const int rc = run_layer(w, x + off, m, out + off, ws, ws_bytes, nullptr, stream, nullptr, nullptr, rev);
    if (rc != MOE_FFN_OK) return rc;
  }
  return MOE_FFN_OK;
}

int moe_ffn_prefill_residual(const moe_ffn_weights* w, const float* x, int32_t n_tokens, float* h,
                             float* xn, float eps, void* ws, size_t ws_bytes,
                             const moe_ffn_routing* routing, hipStream_t stream) {
  const ResidualOut res{h, xn, eps};
  return run_layer(w, x, n_tokens, nullptr, ws, ws_bytes, routing, stream, nullptr, &res);
}

int moe_ffn_prefill_profiled(const moe_ffn_weights* w, const float* x, int32_t n_tokens, float* out,
                             void* ws, size_t ws_bytes, const moe_ffn_routing* routing,
                             hipStream_t stream, hipEvent_t* stage_events) {
  if (!stage_events) return MOE_FFN_INVALID_ARG;
  for (int i = 0; i < MOE_FFN_N_STAGE_EVENTS; ++i)
    if (!stage_events[i]) return MOE_FFN_INVALID_ARG;
  return run_layer(w, x, n_tokens, out, ws, ws_bytes, routing, stream, stage_events);
}

int moe_ffn_decode(const moe_ffn_weights* w, const float* x, int32_t n_tokens, float* out, void* ws,
                   size_t ws_bytes, const moe_ffn_routing* routing, hipStream_t stream) {
  return run_decode(w, x, n_tokens, out, ws, ws_bytes, routing, stream);
}

int moe_ffn_decode_profiled(const moe_ffn_weights* w, const float* x, int32_t n_tokens, float* out,
                            void* ws, size_t ws_bytes, const moe_ffn_routing* routing,
                            hipStream_t stream, hipEvent_t* stage_events) {
  if (!stage_events) return MOE_FFN_INVALID_ARG;
  for (int i = 0; i < MOE_FFN_N_DECODE_STAGE_EVENTS; ++i)
    if (!stage_events[i]) return MOE_FFN_INVALID_ARG;
  return run_decode(w, x, n_tokens, out, ws, ws_bytes, routing, stream, stage_events);
}

int moe_ffn_combine(const float* partial, const float* topk_w, const float* shared_gate, int32_t n,
                    int32_t k, int32_t d, float* out, hipStream_t stream) {
  if (n < 0 || k < 1 || k > MAX_TOPK || d <= 0) return MOE_FFN_INVALID_ARG;
  if (d % 4) return MOE_FFN_UNSUPPORTED;
  if (n == 0) return MOE_FFN_OK;
  if (!partial || !topk_w || !out) return MOE_FFN_INVALID_ARG;
  if (((uintptr_t)partial & 15u) || ((uintptr_t)out & 15u)) return MOE_FFN_UNSUPPORTED;
  const int kk = k + (shared_gate ? 1 : 0);
  const size_t pb = (size_t)n * kk * d * 4, ob = (size_t)n * d * 4;
  if (overlaps(out, ob, partial, pb) || overlaps(out, ob, topk_w, (size_t)n * k * 4) ||
      (shared_gate && overlaps(out, ob, shared_gate, (size_t)n * 4)))
    return MOE_FFN_INVALID_ARG;
  HIP_TRY(launch_combine(partial, topk_w, shared_gate, n, k, kk, d, out, stream));
  return MOE_FFN_OK;
}

int moe_ffn_quantize(const float* v, int64_t n_values, int8_t* q, uint16_t* scales,
                     hipStream_t stream) {
  if (n_values < 0) return MOE_FFN_INVALID_ARG;
  if (n_values % QB) return MOE_FFN_UNSUPPORTED;
  if (n_values == 0) return MOE_FFN_OK;
  if (!v || !q || !scales) return MOE_FFN_INVALID_ARG;
  HIP_TRY(launch_quantize(v, n_values, q, scales, stream));
  return MOE_FFN_OK;
}

int moe_ffn_residual_rmsnorm(float* h, const float* y, float* xn, int32_t n, int32_t d, float eps,
                             hipStream_t stream) {
  if (n < 0 || d <= 0 || !(eps >= 0.0f)) return MOE_FFN_INVALID_ARG;
  if (n == 0) return MOE_FFN_OK;
  if (!h || !xn) return MOE_FFN_INVALID_ARG;
  const size_t b = (size_t)n * d * 4;
  if (overlaps(xn, b, h, b) || (y && overlaps(xn, b, y, b))) return MOE_FFN_INVALID_ARG;
  HIP_TRY(launch_residual_rmsnorm(h, y, xn, n, d, eps, stream));
  return MOE_FFN_OK;
}

int moe_ffn_dbg_block_sums(const moe_ffn_weights* w, void* ws, size_t ws_bytes, int32_t n_tokens,
                           int32_t gemm, int32_t tile, int32_t strip, int32_t kblock, int32_t* sums,
                           int8_t* a_codes, int32_t* info, hipStream_t stream) {
  if (!w || !ws || !sums || !a_codes || !info) return MOE_FFN_INVALID_ARG;
  if (n_tokens < 1 || n_tokens > MAX_TOKENS || (gemm != 0 && gemm != 1)) return MOE_FFN_INVALID_ARG;
  if (w->fmt != MOE_FFN_FMT_Q8_0) return MOE_FFN_UNSUPPORTED;  // reads the Q8_0 code planes
  const Dims& dm = w->dm;
  const WsLayout L = ws_layout(dm, n_tokens);
  if (ws_bytes < L.total) return MOE_FFN_WORKSPACE_TOO_SMALL;
  if ((uintptr_t)ws & 255u) return MOE_FFN_INVALID_ARG;
  // a bound over every group; the kernel checks the tile's own group
  const int strips = gemm == 0 ? dm.kmax_pad / GU_COLS : dm.d_pad / DN_COLS;
  const int kbs = gemm == 0 ? dm.d_pad / QB : dm.kmax_pad / QB;
  if (tile < 0 || tile >= L.tile_bound || strip < 0 || strip >= strips || kblock < 0 || kblock >= kbs)
    return MOE_FFN_INVALID_ARG;
  if (overlaps(sums, 128 * 128 * 4, ws, ws_bytes) || overlaps(a_codes, 128 * 32, ws, ws_bytes) ||
      overlaps(info, 16, ws, ws_bytes) || ((uintptr_t)a_codes & 15u))
    return MOE_FFN_INVALID_ARG;
  const int dev_ok = current_device_matches(w);
  if (dev_ok != MOE_FFN_OK) return dev_ok;
  const GemmArgs a = gemm_args(w, L, (char*)ws, n_tokens);
  HIP_TRY(launch_block_sums(a, gemm == 0, tile, strip, kblock, sums, a_codes, info, stream));
  return MOE_FFN_OK;
}

const char* moe_ffn_status_str(int status) {
  switch (status) {
    case MOE_FFN_OK: return "ok";
    case MOE_FFN_INVALID_ARG: return "invalid argument";
    case MOE_FFN_UNSUPPORTED: return "unsupported shape";
    case MOE_FFN_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_FFN_OUT_OF_MEMORY: return "out of device memory";
    case MOE_FFN_HIP_ERROR: return "HIP runtime error";
    case MOE_FFN_SCRATCH_TOO_SMALL: return "batch exceeds the static scratch of moe_ffn_prefill_static";
    default: return "unknown status";
  }
}

}  // extern "C"
