/*
 * moe_oracle.h -- plain CPU oracle for the batched routed-MoE FFN.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library; the only thing the two sides
 * share is the seeded input generator.
 *
 * Sources (SharpInference GitHub issues):
 *   #406 "batched int8-MMQ trunk prefill gated off for MoE", section "The
 *        work" item 2: batch the router over N tokens, bucket tokens per
 *        expert, grouped expert GEMM, scatter; int8 MMQ with an argmax-stable
 *        contract.
 *   #408 "full-offload MoE decode ~3.4x behind llama.cpp", "Hypothesis":
 *        64 experts / 8 active, norm_topk_prob=false; Q8_1 (int8 block)
 *        activations for the expert matvec; router on the GPU.
 *   #388 "Carnice prefill toward llama.cpp 676 t/s", "Remaining levers" 1:
 *        per-token logits against all expert rows, softmax, top-k and the
 *        shared-expert gate, with the pairs bucketed into the CSR
 *        expStart / expTokI / expTokK.
 *   #129 (batched weighted scatter-reduce), "Scope": per token, sum the na
 *        unweighted down-partials in top-k slot order with the per-(token,
 *        slot) weights, then add the shared-expert row, in that order.
 *
 * Precision: decisions that pick an integer (router top-k, int8 codes) are
 * taken in fp32 exactly as the GPU takes them; every value that is not a
 * decision (softmax weights, the int8 dot products after their exact int32
 * block sums, SwiGLU, the combine) is carried in fp64.  The one exception is
 * ora_combine_f32, which reproduces the fp32 host reduce of #129 bit for bit.
 *
 * Q8_0 weight rows: in/32 blocks of {binary16 scale, int8 q[32]} = 34 bytes,
 * little-endian, unpadded.  Activation blocks: int8 codes plus one binary16
 * scale per 32 values (the Q8_1-style block of #408).
 *
 * Q4_K weight rows (the other MMQ weight format #406 "References" names next
 * to Q8_0; the k-quant super-block of the GGUF format): in/256 super-blocks of
 * 144 bytes = {binary16 d, binary16 dmin, 12 bytes of 6-bit sub-block scales
 * and mins, 128 bytes of 4-bit codes}.  Sub-block j (values 32j..32j+31)
 * holds scale sc_j and min m_j: for j < 4, sc_j = byte j & 63 and m_j =
 * byte j+4 & 63; for j >= 4, sc_j = (byte j+4 & 15) | (byte j-4 >> 6) << 4 and
 * m_j = (byte j+4 >> 4) | (byte j >> 6) << 4 (bytes of the 12).  Code i of
 * sub-block j is the low (j even) or high (j odd) nibble of code byte
 * 32*(j/2) + i.  A value dequantises to d*sc_j*q - dmin*m_j.
 *
 * Q3_K weight rows (the format of the Q3_K expert GEMM #388 "Key references"
 * names; the 3-bit k-quant super-block of the GGUF format): in/256
 * super-blocks of 110 bytes = {32 bytes of high bits, 64 bytes of 2-bit
 * codes, 12 bytes of 6-bit sub-block scales, binary16 d}.  Value i of a
 * super-block (half h = i/128, group g = (i%128)/32, position l = i%32) has
 * the 2-bit code (byte 32h+l of the codes >> 2g) & 3, the high bit = bit
 * 4h+g of high-bit byte l, and q = code - 4 when that bit is clear (q in
 * -4..3).  It belongs to 16-value sub-block s = 8h + 2g + l/16, whose scale
 * sc_s has as low 4 bits nibble s/8 (low nibble first) of scale byte s%8 and
 * as high 2 bits bits 2(s/4), 2(s/4)+1 of scale byte 8 + s%4.  A value
 * dequantises to d*(sc_s - 32)*q.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORA_FMT_Q8_0 0
#define ORA_FMT_Q4_K 1
#define ORA_FMT_Q3_K 2

typedef struct ora_dims {
  int32_t d;              /* hidden size, multiple of 32 (of 256 for Q4_K, Q3_K) */
  int32_t n_experts;      /* E */
  int32_t top_k;          /* k = na */
  int32_t ffn;            /* routed expert intermediate size, multiple of 32 (of 256 for Q4_K, Q3_K) */
  int32_t shared_ffn;     /* shared expert intermediate size, 0 = none */
  int32_t norm_topk_prob; /* 1: renormalise the k selected weights */
  int32_t weight_format;  /* ORA_FMT_Q8_0, ORA_FMT_Q4_K or ORA_FMT_Q3_K: the expert weight rows */
} ora_dims;

/* IEEE binary16 <-> binary32, round to nearest even (n values). */
void ora_half_to_float(const uint16_t* h, float* f, int64_t n);
void ora_float_to_half(const float* f, uint16_t* h, int64_t n);

/* Router logits l[t][e] = sum over j of x[t][j]*W[e][j] in fp32: per block of
 * ORA_ROUTER_BLOCK consecutive j an fmaf chain over ascending j from +0, the
 * block sums added in ascending block order to a total that starts at +0,
 * then + bias[e] (fp32 add) when bias != NULL. */
#define ORA_ROUTER_BLOCK 64
void ora_router_logits(const float* x, int32_t n, int32_t d, const float* w,
                       const float* bias, int32_t n_experts, float* logits);

/* Top-k by (logit descending, expert id ascending); slot s = rank s. */
void ora_topk(const float* logits, int32_t n, int32_t n_experts, int32_t k, int32_t* ids);

/* Softmax over all E logits (fp64), picked at the top-k ids; renormalised
 * over the k picks when norm != 0. */
void ora_route_weights(const float* logits, const int32_t* ids, int32_t n, int32_t n_experts,
                       int32_t k, int32_t norm, double* w);

/* Shared-expert gate: sigmoid(x[t] . g) in fp64. */
void ora_shared_gate(const float* x, int32_t n, int32_t d, const float* g, double* gs);

/* CSR buckets: counts per expert, exclusive scan into exp_start[E+1(+1)],
 * then (token asc, slot asc) placement.  has_shared appends group E holding
 * every token once with slot index k.  exp_start has E+1+has_shared entries;
 * tok_i/tok_k have n*k (+n) entries. */
void ora_csr(const int32_t* ids, int32_t n, int32_t n_experts, int32_t k, int32_t has_shared,
             int32_t* exp_start, int32_t* tok_i, int32_t* tok_k);

/* Per-32-block int8 quantiser (fp32 decisions): amax, code =
 * clamp(rint(v * (127/amax)), -127, 127), scale = binary16(amax/127);
 * an all-zero block gives scale 0 and zero codes. */
void ora_quantize_q8(const float* v, int64_t n_values, int8_t* q, uint16_t* scale16);

/* Q8 dot of an activation row (codes + fp16 scales) with one Q8_0 weight row:
 * sum over blocks of exact int32 block sums times sa*sw, in fp64. */
double ora_q8_dot(const int8_t* qa, const uint16_t* sa16, const uint8_t* w_row, int32_t n_blocks);

/* One Q4_K weight row of in_dim values (in_dim % 256 == 0) dequantised to
 * fp64: out[i] = d*sc_j*q_i - dmin*m_j. */
void ora_q4k_dequant(const uint8_t* w_row, int32_t in_dim, double* out);

/* Q8 activation row (codes + binary16 scales, 32 per block) against one Q4_K
 * weight row of in_dim values: the dot product of the two dequantised rows,
 * sum over i of (sa_b * qa_i) * (d*sc_j*q_i - dmin*m_j), in fp64. */
double ora_q4k_dot(const int8_t* qa, const uint16_t* sa16, const uint8_t* w_row, int32_t in_dim);

/* One Q3_K weight row of in_dim values (in_dim % 256 == 0) dequantised to
 * fp64: out[i] = d*(sc_s - 32)*q_i. */
void ora_q3k_dequant(const uint8_t* w_row, int32_t in_dim, double* out);

/* Q8 activation row against one Q3_K weight row of in_dim values: the dot
 * product of the two dequantised rows, sum over i of (sa_b * qa_i) *
 * (d*(sc_s - 32)*q_i), in fp64. */
double ora_q3k_dot(const int8_t* qa, const uint16_t* sa16, const uint8_t* w_row, int32_t in_dim);

/* The exact int32 sums of one 32-block of an int8 MMQ product (#406
 * "References": Q8_0 MMQ): for activation rows i < m (32 codes each, qa
 * [m][32]) and Q8_0 weight rows j < n (row j starts at w + j * row_bytes),
 *   out[i][j] = sum over t < 32 of qa[i][t] * code t of block kblock of row j.
 * No scale enters: these are the integers the scaled block products are
 * formed from. */
void ora_q8_block_sums(const int8_t* qa, int32_t m, const uint8_t* w, int32_t n, int64_t row_bytes,
                       int32_t kblock, int32_t* out);

/* One SwiGLU expert on one quantised token row: g,u = Q8 dots; h = silu(g)*u
 * (fp64), requantised per 32 in fp32; y = Q8 dot with the down rows.
 * gate/up: [ffn][d/32*34] bytes, down: [d][ffn/32*34] bytes.  hq/hs/h may be
 * NULL. */
void ora_expert_ffn(int32_t d, int32_t ffn, const int8_t* xq, const uint16_t* xs,
                    const uint8_t* gate, const uint8_t* up, const uint8_t* down, double* y,
                    int8_t* hq, uint16_t* hs, double* h);

/* ora_expert_ffn with the expert weight rows in format fmt (ORA_FMT_*):
 * gate/up rows of d values, down rows of ffn values. */
void ora_expert_ffn_fmt(int32_t fmt, int32_t d, int32_t ffn, const int8_t* xq, const uint16_t* xs,
                        const uint8_t* gate, const uint8_t* up, const uint8_t* down, double* y,
                        int8_t* hq, uint16_t* hs, double* h);

/* The per-token loop over the listed tokens (OpenMP over the list):
 * router, top-k, weights, quantiser, k experts (+ shared), combine in fp64.
 * out: [n_list][d].  partial (may be NULL): [n_list][k+has_shared][d]
 * unweighted expert outputs.  ids/w/gs (may be NULL): [n_list][k], [n_list][k],
 * [n_list].  Returns 0, or -1 on a bad argument. */
int32_t ora_moe_tokens(const ora_dims* dm, const float* x, int32_t n_tokens,
                       const float* router_w, const float* router_bias,
                       const uint8_t* gate_q8, const uint8_t* up_q8, const uint8_t* down_q8,
                       const uint8_t* sh_gate_q8, const uint8_t* sh_up_q8, const uint8_t* sh_down_q8,
                       const float* sh_gate_vec, const int32_t* token_list, int32_t n_list,
                       double* out, double* partial, int32_t* ids, double* w, double* gs);

/* The same layer evaluated grouped by expert: router for all tokens, CSR,
 * then every expert group's rows in CSR order, then the combine.  Must agree
 * bit for bit with ora_moe_tokens.  out: [n_tokens][d]. */
int32_t ora_moe_grouped(const ora_dims* dm, const float* x, int32_t n_tokens,
                        const float* router_w, const float* router_bias,
                        const uint8_t* gate_q8, const uint8_t* up_q8, const uint8_t* down_q8,
                        const uint8_t* sh_gate_q8, const uint8_t* sh_up_q8, const uint8_t* sh_down_q8,
                        const float* sh_gate_vec, double* out);

/* The fp32 host reduce of #129: o = +0; o = fmaf(w[t][s], P[t][s][j], o) for
 * s = 0..k-1; then o = fmaf(gs[t], P[t][k][j], o) when gs != NULL.
 * partial: [n][kk][d] with kk = k (+1 with a shared row). */
void ora_combine_f32(const float* partial, const float* w, const float* gs, int32_t n, int32_t k,
                     int32_t kk, int32_t d, float* out);

/* Number of OpenMP threads the parallel loops above use. */
int32_t ora_num_threads(void);
/* Set the number of host threads later calls use (timing only; no effect on
 * any result: every token is evaluated by one thread). */
void ora_set_num_threads(int32_t n);

/* RMSNorm with unit gain in fp64: x / sqrt(mean(x^2) + eps). */
void ora_rmsnorm(const float* x, int32_t n, int32_t d, double eps, double* out);

#ifdef __cplusplus
}
#endif
#endif
