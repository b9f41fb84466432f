/*
 * moe_oracle.c -- plain, slow CPU oracle for the batched routed-MoE FFN.
 *
 * TEST INFRASTRUCTURE: see moe_oracle.h.  Built with gcc -O2
 * -ffp-contract=off (no fast-math) so that every fp32 operation written here
 * is the one executed; fmaf() is used wherever a fused multiply-add is meant.
 *
 * The layer, following the SharpInference issue pages:
 *   1. router logits over all experts, top-k, softmax weights
 *      (#388 "Remaining levers" 1; #408 "Hypothesis": norm_topk_prob);
 *   2. per-expert buckets in CSR form expStart/expTokI/expTokK (#388 lever 1,
 *      #406 "The work" 2);
 *   3. int8 (Q8_0 weight x int8 block activation) expert GEMMs: gate/up, SwiGLU,
 *      down, giving unweighted down-partials (#406 "The work" 2 and
 *      "References" (Q8_0 MMQ); #408 lever 2 (Q8_1 activations); #129
 *      opening paragraph (routed-expert gate/up/down));
 *   4. the weighted combine in top-k slot order plus the shared row
 *      (#129 "Scope").
 */
#include "moe_oracle.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

#define QB 32
#define QBYTES 34
#define Q4K_VALUES 256 /* values per Q4_K super-block */
#define Q4K_BYTES 144  /* bytes per Q4_K super-block */
#define Q3K_BYTES 110  /* bytes per Q3_K super-block (256 values) */

/* ---------------------------------------------------------------- fp16 */
/* IEEE 754 binary16 decoding: sign, 5-bit exponent (bias 15), 10-bit fraction. */
static float half_bits_to_float(uint16_t h) {
  uint32_t sign = ((uint32_t)h & 0x8000u) << 16;
  uint32_t ex = ((uint32_t)h >> 10) & 0x1fu;
  uint32_t fr = (uint32_t)h & 0x3ffu;
  uint32_t bits;
  float f;
  if (ex == 0) {
    /* zero or subnormal: fr * 2^-24, exact in binary32 */
    f = (float)fr * 5.9604644775390625e-8f;
    return sign ? -f : f;
  }
  if (ex == 31)
    bits = sign | 0x7f800000u | (fr << 13);
  else
    bits = sign | ((ex - 15u + 127u) << 23) | (fr << 13);
  memcpy(&f, &bits, 4);
  return f;
}

/* binary32 -> binary16 with round-to-nearest-even. */
static uint16_t float_to_half_bits(float f) {
  uint32_t x;
  memcpy(&x, &f, 4);
  uint32_t sign = (x >> 16) & 0x8000u;
  uint32_t ax = x & 0x7fffffffu;
  if (ax >= 0x7f800000u) /* inf / nan */
    return (uint16_t)(sign | 0x7c00u | (ax > 0x7f800000u ? 0x200u : 0u));
  if (ax >= 0x477ff000u) /* >= 65520 rounds past 65504 to inf */
    return (uint16_t)(sign | 0x7c00u);
  if (ax < 0x38800000u) {
    /* below 2^-14: a binary16 subnormal (or zero); unit 2^-24.  Scaling by
     * 2^24 is exact, rintf rounds to nearest even; 1024 lands on the
     * smallest normal, which has the same bit pattern. */
    float a;
    memcpy(&a, &ax, 4);
    uint32_t m = (uint32_t)rintf(a * 16777216.0f);
    return (uint16_t)(sign | m);
  }
  uint32_t ex = (ax >> 23) - 127u + 15u;
  uint32_t fr = ax & 0x7fffffu;
  uint32_t h = (ex << 10) | (fr >> 13);
  uint32_t rem = fr & 0x1fffu;
  if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1u; /* carry may bump the exponent */
  return (uint16_t)(sign | h);
}

void ora_half_to_float(const uint16_t* h, float* f, int64_t n) {
  for (int64_t i = 0; i < n; ++i) f[i] = half_bits_to_float(h[i]);
}

void ora_float_to_half(const float* f, uint16_t* h, int64_t n) {
  for (int64_t i = 0; i < n; ++i) h[i] = float_to_half_bits(f[i]);
}

/* -------------------------------------------------------------- router */
/* #388, "Remaining levers" 1: the logits of every token against every
 * expert's router row, in fp32 and in one fixed order (the pages fix none):
 * j is cut into blocks of ORA_ROUTER_BLOCK; each block's products are
 * summed by a chain of fused multiply-adds over ascending j from +0, and the
 * block sums are added one by one in ascending block order. */
void ora_router_logits(const float* x, int32_t n, int32_t d, const float* w,
                       const float* bias, int32_t n_experts, float* logits) {
  for (int32_t t = 0; t < n; ++t) {
    const float* xr = x + (int64_t)t * d;
    for (int32_t e = 0; e < n_experts; ++e) {
      const float* wr = w + (int64_t)e * d;
      float total = 0.0f;
      for (int32_t j0 = 0; j0 < d; j0 += ORA_ROUTER_BLOCK) {
        const int32_t j1 = j0 + ORA_ROUTER_BLOCK < d ? j0 + ORA_ROUTER_BLOCK : d;
        float block = 0.0f;
        for (int32_t j = j0; j < j1; ++j) block = fmaf(xr[j], wr[j], block);
        total = total + block;
      }
      if (bias) total = total + bias[e];
      logits[(int64_t)t * n_experts + e] = total;
    }
  }
}

/* a outranks b: larger logit first, lower id on equal logits. */
static int outranks(float la, int32_t a, float lb, int32_t b) {
  return la > lb || (la == lb && a < b);
}

/* Top-k selection by repeated best-of-the-rest; slot s holds the rank-s expert. */
void ora_topk(const float* logits, int32_t n, int32_t n_experts, int32_t k, int32_t* ids) {
  unsigned char* taken = (unsigned char*)malloc((size_t)n_experts);
  for (int32_t t = 0; t < n; ++t) {
    const float* l = logits + (int64_t)t * n_experts;
    memset(taken, 0, (size_t)n_experts);
    for (int32_t s = 0; s < k; ++s) {
      int32_t best = -1;
      for (int32_t e = 0; e < n_experts; ++e) {
        if (taken[e]) continue;
        if (best < 0 || outranks(l[e], e, l[best], best)) best = e;
      }
      taken[best] = 1;
      ids[(int64_t)t * k + s] = best;
    }
  }
  free(taken);
}

/* Softmax over all experts, read at the selected ids (norm_topk_prob=false,
 * #408); with norm != 0 the k picks are divided by their sum. */
void ora_route_weights(const float* logits, const int32_t* ids, int32_t n, int32_t n_experts,
                       int32_t k, int32_t norm, double* w) {
  for (int32_t t = 0; t < n; ++t) {
    const float* l = logits + (int64_t)t * n_experts;
    double m = (double)l[0];
    for (int32_t e = 1; e < n_experts; ++e)
      if ((double)l[e] > m) m = (double)l[e];
    double den = 0.0;
    for (int32_t e = 0; e < n_experts; ++e) den += exp((double)l[e] - m);
    double sum = 0.0;
    for (int32_t s = 0; s < k; ++s) {
      double p = exp((double)l[ids[(int64_t)t * k + s]] - m) / den;
      w[(int64_t)t * k + s] = p;
      sum += p;
    }
    if (norm)
      for (int32_t s = 0; s < k; ++s) w[(int64_t)t * k + s] /= sum;
  }
}

/* "shexp-gate" (#388 router phase): a scalar sigmoid gate per token. */
void ora_shared_gate(const float* x, int32_t n, int32_t d, const float* g, double* gs) {
  for (int32_t t = 0; t < n; ++t) {
    double acc = 0.0;
    for (int32_t j = 0; j < d; ++j) acc += (double)x[(int64_t)t * d + j] * (double)g[j];
    gs[t] = 1.0 / (1.0 + exp(-acc));
  }
}

/* ----------------------------------------------------------------- CSR */
/* #388 lever 1: expStart / expTokI / expTokK.  Counting sort; within an
 * expert the pairs keep (token, slot) order. */
void ora_csr(const int32_t* ids, int32_t n, int32_t n_experts, int32_t k, int32_t has_shared,
             int32_t* exp_start, int32_t* tok_i, int32_t* tok_k) {
  int32_t* cur = (int32_t*)calloc((size_t)n_experts + 1, sizeof(int32_t));
  for (int64_t p = 0; p < (int64_t)n * k; ++p) cur[ids[p]] += 1;
  int32_t run = 0;
  for (int32_t e = 0; e < n_experts; ++e) {
    int32_t c = cur[e];
    exp_start[e] = run;
    cur[e] = run;
    run += c;
  }
  exp_start[n_experts] = run;
  for (int32_t t = 0; t < n; ++t)
    for (int32_t s = 0; s < k; ++s) {
      int32_t e = ids[(int64_t)t * k + s];
      int32_t p = cur[e]++;
      tok_i[p] = t;
      tok_k[p] = s;
    }
  if (has_shared) {
    for (int32_t t = 0; t < n; ++t) {
      tok_i[run + t] = t;
      tok_k[run + t] = k;
    }
    exp_start[n_experts + 1] = run + n;
  }
  free(cur);
}

/* ----------------------------------------------------------- quantiser */
/* Per-32-block int8 activations (#408 lever 2, Q8_1-style): all decisions in
 * fp32 -- amax, the reciprocal 127/amax, the product, round-half-even. */
void ora_quantize_q8(const float* v, int64_t n_values, int8_t* q, uint16_t* scale16) {
  for (int64_t b = 0; b < n_values / QB; ++b) {
    const float* vb = v + b * QB;
    float amax = 0.0f;
    for (int i = 0; i < QB; ++i) {
      float a = fabsf(vb[i]);
      if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
      scale16[b] = 0;
      for (int i = 0; i < QB; ++i) q[b * QB + i] = 0;
      continue;
    }
    float dd = amax / 127.0f;
    float id = 127.0f / amax;
    scale16[b] = float_to_half_bits(dd);
    for (int i = 0; i < QB; ++i) {
      float r = rintf(vb[i] * id);
      if (r > 127.0f) r = 127.0f;
      if (r < -127.0f) r = -127.0f;
      q[b * QB + i] = (int8_t)r;
    }
  }
}

/* ------------------------------------------------------------- Q8 dot */
/* int8 MMQ semantics (#406 "References": Q8_0 MMQ): exact int32 sum per
 * 32-block, scaled by activation-scale * weight-scale, summed in fp64. */
double ora_q8_dot(const int8_t* qa, const uint16_t* sa16, const uint8_t* w_row, int32_t n_blocks) {
  double acc = 0.0;
  for (int32_t b = 0; b < n_blocks; ++b) {
    const uint8_t* blk = w_row + (int64_t)b * QBYTES;
    uint16_t d16 = (uint16_t)(blk[0] | (blk[1] << 8));
    const int8_t* qw = (const int8_t*)(blk + 2);
    int32_t c = 0;
    for (int i = 0; i < QB; ++i) c += (int32_t)qa[(int64_t)b * QB + i] * (int32_t)qw[i];
    double s = (double)half_bits_to_float(sa16[b]) * (double)half_bits_to_float(d16);
    acc += (double)c * s;
  }
  return acc;
}

/* The integer core of the int8 MMQ product, one block at a time: the same
 * exact int32 block sum ora_q8_dot forms, for a grid of rows. */
void ora_q8_block_sums(const int8_t* qa, int32_t m, const uint8_t* w, int32_t n, int64_t row_bytes,
                       int32_t kblock, int32_t* out) {
  for (int32_t i = 0; i < m; ++i)
    for (int32_t j = 0; j < n; ++j) {
      const int8_t* qw = (const int8_t*)(w + (int64_t)j * row_bytes + (int64_t)kblock * QBYTES + 2);
      int32_t c = 0;
      for (int t = 0; t < QB; ++t) c += (int32_t)qa[(int64_t)i * QB + t] * (int32_t)qw[t];
      out[(int64_t)i * n + j] = c;
    }
}

/* ------------------------------------------------------------- Q4_K */
/* Scale and min of sub-block j from the 12 packed bytes (moe_oracle.h). */
static void q4k_scale_min(const uint8_t* s12, int j, int* sc, int* m) {
  if (j < 4) {
    *sc = s12[j] & 63;
    *m = s12[j + 4] & 63;
  } else {
    *sc = (s12[j + 4] & 15) | ((s12[j - 4] >> 6) << 4);
    *m = (s12[j + 4] >> 4) | ((s12[j] >> 6) << 4);
  }
}

/* The 256 values of one super-block, dequantised in fp64: value i of
 * sub-block j is d * sc_j * q_i - dmin * m_j. */
static void q4k_super_block(const uint8_t* blk, double* out) {
  const double d = (double)half_bits_to_float((uint16_t)(blk[0] | (blk[1] << 8)));
  const double dmin = (double)half_bits_to_float((uint16_t)(blk[2] | (blk[3] << 8)));
  for (int j = 0; j < 8; ++j) {
    int sc, m;
    q4k_scale_min(blk + 4, j, &sc, &m);
    for (int t = 0; t < 32; ++t) {
      const uint8_t byte = blk[16 + 32 * (j / 2) + t];
      const int q = (j & 1) ? (byte >> 4) : (byte & 15);
      out[32 * j + t] = d * (double)sc * (double)q - dmin * (double)m;
    }
  }
}

void ora_q4k_dequant(const uint8_t* w_row, int32_t in_dim, double* out) {
  for (int32_t s = 0; s < in_dim / Q4K_VALUES; ++s) q4k_super_block(w_row + (int64_t)s * Q4K_BYTES, out + (int64_t)s * Q4K_VALUES);
}

/* Q4_K MMQ (#406 "References"): the product of the dequantised activation
 * and weight rows, written as its definition (the sum over ascending i). */
double ora_q4k_dot(const int8_t* qa, const uint16_t* sa16, const uint8_t* w_row, int32_t in_dim) {
  double acc = 0.0;
  double w[Q4K_VALUES];
  for (int32_t s = 0; s < in_dim / Q4K_VALUES; ++s) {
    q4k_super_block(w_row + (int64_t)s * Q4K_BYTES, w);
    for (int32_t b = 0; b < Q4K_VALUES / QB; ++b) {
      const int32_t i0 = s * Q4K_VALUES + b * QB;
      const double sa = (double)half_bits_to_float(sa16[i0 / QB]);
      for (int32_t t = 0; t < QB; ++t) {
        const double a = sa * (double)qa[i0 + t];
        acc += a * w[b * QB + t];
      }
    }
  }
  return acc;
}

/* ------------------------------------------------------------- Q3_K */
/* The 256 values of one Q3_K super-block, dequantised in fp64 (layout in
 * moe_oracle.h): value i = d * (sc_s - 32) * q_i. */
static void q3k_super_block(const uint8_t* blk, double* out) {
  const uint8_t* hbits = blk;
  const uint8_t* codes = blk + 32;
  const uint8_t* sc = blk + 96;
  const double d = (double)half_bits_to_float((uint16_t)(blk[108] | (blk[109] << 8)));
  for (int i = 0; i < Q4K_VALUES; ++i) {
    const int h = i / 128, g = (i % 128) / 32, l = i % 32;
    const int code = (codes[32 * h + l] >> (2 * g)) & 3;
    const int high = (hbits[l] >> (4 * h + g)) & 1;
    const int q = high ? code : code - 4;
    const int s = 8 * h + 2 * g + l / 16;
    const int lo4 = (sc[s % 8] >> (4 * (s / 8))) & 15;
    const int hi2 = (sc[8 + s % 4] >> (2 * (s / 4))) & 3;
    const int scale = lo4 | (hi2 << 4);
    out[i] = d * (double)(scale - 32) * (double)q;
  }
}

void ora_q3k_dequant(const uint8_t* w_row, int32_t in_dim, double* out) {
  for (int32_t s = 0; s < in_dim / Q4K_VALUES; ++s) q3k_super_block(w_row + (int64_t)s * Q3K_BYTES, out + (int64_t)s * Q4K_VALUES);
}

/* The product of the dequantised activation and Q3_K weight rows, written
 * as its definition (the sum over ascending i). */
double ora_q3k_dot(const int8_t* qa, const uint16_t* sa16, const uint8_t* w_row, int32_t in_dim) {
  double acc = 0.0;
  double w[Q4K_VALUES];
  for (int32_t s = 0; s < in_dim / Q4K_VALUES; ++s) {
    q3k_super_block(w_row + (int64_t)s * Q3K_BYTES, w);
    for (int32_t b = 0; b < Q4K_VALUES / QB; ++b) {
      const int32_t i0 = s * Q4K_VALUES + b * QB;
      const double sa = (double)half_bits_to_float(sa16[i0 / QB]);
      for (int32_t t = 0; t < QB; ++t) {
        const double a = sa * (double)qa[i0 + t];
        acc += a * w[b * QB + t];
      }
    }
  }
  return acc;
}

/* Bytes of one weight row of in_dim values and the dot product of format fmt. */
static int64_t row_bytes_of(int32_t fmt, int32_t in_dim) {
  if (fmt == ORA_FMT_Q4_K) return (int64_t)(in_dim / Q4K_VALUES) * Q4K_BYTES;
  if (fmt == ORA_FMT_Q3_K) return (int64_t)(in_dim / Q4K_VALUES) * Q3K_BYTES;
  return (int64_t)(in_dim / QB) * QBYTES;
}
static double wdot(int32_t fmt, const int8_t* qa, const uint16_t* sa16, const uint8_t* w_row, int32_t in_dim) {
  if (fmt == ORA_FMT_Q4_K) return ora_q4k_dot(qa, sa16, w_row, in_dim);
  if (fmt == ORA_FMT_Q3_K) return ora_q3k_dot(qa, sa16, w_row, in_dim);
  return ora_q8_dot(qa, sa16, w_row, in_dim / QB);
}

/* ------------------------------------------------------------- expert */
/* Routed-expert gate/up/down (#129 opening paragraph): h = silu(gate) * up,
 * requantised per 32 for the int8 down GEMM; y is the unweighted partial. */
void ora_expert_ffn_fmt(int32_t fmt, int32_t d, int32_t ffn, const int8_t* xq, const uint16_t* xs,
                        const uint8_t* gate, const uint8_t* up, const uint8_t* down, double* y,
                        int8_t* hq, uint16_t* hs, double* h) {
  const int32_t nbf = ffn / QB;
  const int64_t row_d = row_bytes_of(fmt, d), row_f = row_bytes_of(fmt, ffn);
  float* hf = (float*)malloc(sizeof(float) * (size_t)ffn);
  int8_t* q = (int8_t*)malloc((size_t)ffn);
  uint16_t* sc = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)nbf);
  for (int32_t i = 0; i < ffn; ++i) {
    double g = wdot(fmt, xq, xs, gate + i * row_d, d);
    double u = wdot(fmt, xq, xs, up + i * row_d, d);
    double hv = g / (1.0 + exp(-g)) * u;
    if (h) h[i] = hv;
    hf[i] = (float)hv;
  }
  ora_quantize_q8(hf, ffn, q, sc);
  for (int32_t j = 0; j < d; ++j) y[j] = wdot(fmt, q, sc, down + j * row_f, ffn);
  if (hq) memcpy(hq, q, (size_t)ffn);
  if (hs) memcpy(hs, sc, sizeof(uint16_t) * (size_t)nbf);
  free(hf);
  free(q);
  free(sc);
}

void ora_expert_ffn(int32_t d, int32_t ffn, const int8_t* xq, const uint16_t* xs,
                    const uint8_t* gate, const uint8_t* up, const uint8_t* down, double* y,
                    int8_t* hq, uint16_t* hs, double* h) {
  ora_expert_ffn_fmt(ORA_FMT_Q8_0, d, ffn, xq, xs, gate, up, down, y, hq, hs, h);
}

static int dims_ok(const ora_dims* dm) {
  if (!dm) return 0;
  if (dm->weight_format != ORA_FMT_Q8_0 && dm->weight_format != ORA_FMT_Q4_K && dm->weight_format != ORA_FMT_Q3_K)
    return 0;
  const int32_t unit = dm->weight_format == ORA_FMT_Q8_0 ? QB : Q4K_VALUES;
  if (dm->d <= 0 || dm->d % unit || dm->ffn <= 0 || dm->ffn % unit) return 0;
  if (dm->shared_ffn < 0 || dm->shared_ffn % unit) return 0;
  if (dm->n_experts <= 0 || dm->top_k <= 0 || dm->top_k > dm->n_experts) return 0;
  return 1;
}

/* --------------------------------------------------------- whole layer */
/* The per-token loop: each listed token runs router -> top-k -> weights ->
 * quantiser -> its k experts (+ shared) -> combine, independently. */
int32_t ora_moe_tokens(const ora_dims* dm, const float* x, int32_t n_tokens,
                       const float* router_w, const float* router_bias,
                       const uint8_t* gate_q8, const uint8_t* up_q8, const uint8_t* down_q8,
                       const uint8_t* sh_gate_q8, const uint8_t* sh_up_q8, const uint8_t* sh_down_q8,
                       const float* sh_gate_vec, const int32_t* token_list, int32_t n_list,
                       double* out, double* partial, int32_t* ids_out, double* w_out,
                       double* gs_out) {
  if (!dims_ok(dm) || !x || !router_w || !gate_q8 || !up_q8 || !down_q8 || !out) return -1;
  const int32_t d = dm->d, E = dm->n_experts, k = dm->top_k, F = dm->ffn, Fs = dm->shared_ffn;
  const int has_sh = Fs > 0;
  if (has_sh && (!sh_gate_q8 || !sh_up_q8 || !sh_down_q8 || !sh_gate_vec)) return -1;
  for (int32_t i = 0; i < n_list; ++i)
    if (token_list[i] < 0 || token_list[i] >= n_tokens) return -1;
  const int32_t kk = k + has_sh, fmt = dm->weight_format;
  const int64_t ex_gu = (int64_t)F * row_bytes_of(fmt, d);  /* bytes per expert, gate or up */
  const int64_t ex_dn = (int64_t)d * row_bytes_of(fmt, F);  /* bytes per expert, down */

#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t i = 0; i < n_list; ++i) {
    const int32_t t = token_list[i];
    const float* xt = x + (int64_t)t * d;
    float* logits = (float*)malloc(sizeof(float) * (size_t)E);
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    double* w = (double*)malloc(sizeof(double) * (size_t)k);
    int8_t* xq = (int8_t*)malloc((size_t)d);
    uint16_t* xs = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(d / QB));
    double* y = (double*)malloc(sizeof(double) * (size_t)d * (size_t)kk);

    ora_router_logits(xt, 1, d, router_w, router_bias, E, logits);
    ora_topk(logits, 1, E, k, ids);
    ora_route_weights(logits, ids, 1, E, k, dm->norm_topk_prob, w);
    ora_quantize_q8(xt, d, xq, xs);
    for (int32_t s = 0; s < k; ++s) {
      int32_t e = ids[s];
      ora_expert_ffn_fmt(fmt, d, F, xq, xs, gate_q8 + e * ex_gu, up_q8 + e * ex_gu, down_q8 + e * ex_dn,
                         y + (int64_t)s * d, NULL, NULL, NULL);
    }
    double gs = 0.0;
    if (has_sh) {
      ora_shared_gate(xt, 1, d, sh_gate_vec, &gs);
      ora_expert_ffn_fmt(fmt, d, Fs, xq, xs, sh_gate_q8, sh_up_q8, sh_down_q8, y + (int64_t)k * d, NULL,
                         NULL, NULL);
    }
    /* #129 "Scope": slot order k = 0..na-1, then the shared row. */
    for (int32_t j = 0; j < d; ++j) {
      double o = 0.0;
      for (int32_t s = 0; s < k; ++s) o += w[s] * y[(int64_t)s * d + j];
      if (has_sh) o += gs * y[(int64_t)k * d + j];
      out[(int64_t)i * d + j] = o;
    }
    if (partial) memcpy(partial + (int64_t)i * kk * d, y, sizeof(double) * (size_t)kk * (size_t)d);
    if (ids_out) memcpy(ids_out + (int64_t)i * k, ids, sizeof(int32_t) * (size_t)k);
    if (w_out) memcpy(w_out + (int64_t)i * k, w, sizeof(double) * (size_t)k);
    if (gs_out) gs_out[i] = gs;
    free(logits);
    free(ids);
    free(w);
    free(xq);
    free(xs);
    free(y);
  }
  return 0;
}

/* The grouped evaluation: the same expert function applied expert by expert
 * over the CSR rows (#406 "The work" 2: gather per expert, GEMM, scatter). */
int32_t ora_moe_grouped(const ora_dims* dm, const float* x, int32_t n_tokens,
                        const float* router_w, const float* router_bias,
                        const uint8_t* gate_q8, const uint8_t* up_q8, const uint8_t* down_q8,
                        const uint8_t* sh_gate_q8, const uint8_t* sh_up_q8, const uint8_t* sh_down_q8,
                        const float* sh_gate_vec, double* out) {
  if (!dims_ok(dm) || !x || !router_w || !gate_q8 || !up_q8 || !down_q8 || !out) return -1;
  const int32_t d = dm->d, E = dm->n_experts, k = dm->top_k, F = dm->ffn, Fs = dm->shared_ffn;
  const int has_sh = Fs > 0;
  if (has_sh && (!sh_gate_q8 || !sh_up_q8 || !sh_down_q8 || !sh_gate_vec)) return -1;
  const int32_t N = n_tokens, kk = k + has_sh, fmt = dm->weight_format;
  const int64_t ex_gu = (int64_t)F * row_bytes_of(fmt, d);
  const int64_t ex_dn = (int64_t)d * row_bytes_of(fmt, F);

  float* logits = (float*)malloc(sizeof(float) * (size_t)N * E + 1);
  int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)N * k + 1);
  double* w = (double*)malloc(sizeof(double) * (size_t)N * k + 1);
  double* gs = (double*)calloc((size_t)N + 1, sizeof(double));
  int8_t* xq = (int8_t*)malloc((size_t)N * d + 1);
  uint16_t* xs = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)N * (d / QB) + 1);
  int32_t* start = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E + 2));
  int32_t* tok_i = (int32_t*)malloc(sizeof(int32_t) * (size_t)N * kk + 1);
  int32_t* tok_k = (int32_t*)malloc(sizeof(int32_t) * (size_t)N * kk + 1);
  double* part = (double*)malloc(sizeof(double) * (size_t)N * kk * d + 1);

  ora_router_logits(x, N, d, router_w, router_bias, E, logits);
  ora_topk(logits, N, E, k, ids);
  ora_route_weights(logits, ids, N, E, k, dm->norm_topk_prob, w);
  if (has_sh) ora_shared_gate(x, N, d, sh_gate_vec, gs);
  ora_quantize_q8(x, (int64_t)N * d, xq, xs);
  ora_csr(ids, N, E, k, has_sh, start, tok_i, tok_k);

  for (int32_t g = 0; g < E + has_sh; ++g) {
    const int shared = (g == E);
    const int32_t Fg = shared ? Fs : F;
    const uint8_t* gw = shared ? sh_gate_q8 : gate_q8 + g * ex_gu;
    const uint8_t* uw = shared ? sh_up_q8 : up_q8 + g * ex_gu;
    const uint8_t* dw = shared ? sh_down_q8 : down_q8 + g * ex_dn;
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t p = start[g]; p < start[g + 1]; ++p) {
      int32_t t = tok_i[p], s = tok_k[p];
      ora_expert_ffn_fmt(fmt, d, Fg, xq + (int64_t)t * d, xs + (int64_t)t * (d / QB), gw, uw, dw,
                         part + ((int64_t)t * kk + s) * d, NULL, NULL, NULL);
    }
  }
  for (int32_t t = 0; t < N; ++t)
    for (int32_t j = 0; j < d; ++j) {
      double o = 0.0;
      for (int32_t s = 0; s < k; ++s) o += w[(int64_t)t * k + s] * part[((int64_t)t * kk + s) * d + j];
      if (has_sh) o += gs[t] * part[((int64_t)t * kk + k) * d + j];
      out[(int64_t)t * d + j] = o;
    }
  free(logits);
  free(ids);
  free(w);
  free(gs);
  free(xq);
  free(xs);
  free(start);
  free(tok_i);
  free(tok_k);
  free(part);
  return 0;
}

/* #129 "Scope": the sequential host reduce, Clear -> AddScaledInPlace per slot
 * in top-k order -> AddInPlace(shared), in fp32.  Each scaled add is one fused
 * multiply-add; the shared row enters through its gate. */
void ora_combine_f32(const float* partial, const float* w, const float* gs, int32_t n, int32_t k,
                     int32_t kk, int32_t d, float* out) {
  for (int32_t t = 0; t < n; ++t)
    for (int32_t j = 0; j < d; ++j) {
      float o = 0.0f;
      for (int32_t s = 0; s < k; ++s)
        o = fmaf(w[(int64_t)t * k + s], partial[((int64_t)t * kk + s) * d + j], o);
      if (gs) o = fmaf(gs[t], partial[((int64_t)t * kk + k) * d + j], o);
      out[(int64_t)t * d + j] = o;
    }
}

void ora_rmsnorm(const float* x, int32_t n, int32_t d, double eps, double* out) {
  for (int32_t t = 0; t < n; ++t) {
    double ss = 0.0;
    for (int32_t j = 0; j < d; ++j) ss += (double)x[(int64_t)t * d + j] * (double)x[(int64_t)t * d + j];
    double r = 1.0 / sqrt(ss / d + eps);
    for (int32_t j = 0; j < d; ++j) out[(int64_t)t * d + j] = (double)x[(int64_t)t * d + j] * r;
  }
}

int32_t ora_num_threads(void) { return (int32_t)omp_get_max_threads(); }

void ora_set_num_threads(int32_t n) {
  if (n >= 1) omp_set_num_threads(n);
}
