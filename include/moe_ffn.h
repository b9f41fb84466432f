/*
 * moe_ffn.h -- C ABI of the MI355X (gfx950) batched routed-MoE FFN library
 * (libmoe_ffn.so).
 *
 * The operation is the batched MoE FFN over N prompt tokens described in the
 * SharpInference issue pages:
 *   #406 "batched int8-MMQ trunk prefill gated off for MoE", "The work" item 2:
 *        batch the router over N tokens, group tokens per expert, run a
 *        grouped/segmented expert GEMM, scatter the results back;
 *        "argmax-stable (int8 MMQ)" is the accepted numeric contract;
 *   #388 "Carnice prefill toward llama.cpp 676 t/s", "Remaining levers" 1:
 *        routing (logits, softmax, top-k, shared-expert gate) and the
 *        expStart / expTokI / expTokK bucketing both run on the device, so
 *        no routing data crosses to the host inside a call;
 *   #408 "full-offload MoE decode", "Hypothesis": 64 experts / 8 active,
 *        norm_topk_prob=false; one fused gathered-expert launch instead of
 *        per-expert matvecs; int8 (Q8_1-style) activations;
 *   #129 (batched weighted scatter-reduce), "Scope": per token, the na
 *        unweighted down-partials are summed in top-k slot order with their
 *        weights, then the shared-expert row is added, in one launch over
 *        N x embDim.
 *
 * Numerics (what every entry point computes):
 *   logit[t][e]  = fp32 sum of x[t][j] * router_w[e][j] in blocks of 64 j:
 *                  per block a fused multiply-add chain over ascending j
 *                  from +0, the block sums added in ascending block order
 *                  to a total from +0, then + bias[e];
 *   top-k        = experts by (logit descending, id ascending); slot s = rank s;
 *   w[t][s]      = softmax over all E logits at ids[t][s]; divided by the sum
 *                  of the k picks when norm_topk_prob;
 *   gs[t]        = sigmoid(x[t] . shared_gate_vec) when a shared expert exists;
 *   activations  = per-32-block int8 codes rint(x * 127/amax) (half to even)
 *                  with a binary16 scale amax/127; zero block -> zeros;
 *   expert FFN   = g, u = int8 block dot products (exact int32 per block,
 *                  times activation-scale * weight-scale, summed in fp32);
 *                  h = silu(g) * u, requantised per 32 like the activations;
 *                  y = int8 dot of h with the down rows (unweighted partial);
 *   out[t][j]    = fp32 fused multiply-add chain from +0 over s = 0..k-1 of
 *                  w[t][s] * y_s[j], then gs[t] * shared_y[j] when present.
 *
 * Conventions:
 *   - Every pointer argument is a DEVICE pointer unless stated otherwise.
 *     Struct arguments (dims, routing) are host memory.
 *   - Every call returns a moe_ffn_status.  Arguments are validated on the
 *     host before anything is enqueued; on an error nothing is enqueued.  The
 *     library never aborts and never throws.
 *   - Work is enqueued on the caller's stream and the call returns without a
 *     host synchronisation, except moe_ffn_weights_create, which synchronises
 *     its stream before returning.  Device faults surface at the caller's next
 *     synchronisation.
 *   - A weights handle is immutable after creation and may be shared by
 *     concurrent calls; concurrent calls need their own workspaces.
 *   - Supported shapes: d, ffn, shared_ffn multiples of 32 (internally
 *     zero-padded to multiples of 128); 1 <= n_experts <= 256;
 *     1 <= top_k <= min(n_experts, 16); 0 <= n_tokens <= the max_tokens the
 *     workspace was sized for, and n_tokens * padded d below 2^32 (the
 *     activation codes of one call are addressed by 32-bit offsets); other
 *     counts are MOE_FFN_INVALID_ARG.  n_tokens == 0 is a no-op.
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_ffn_status {
  MOE_FFN_OK = 0,
  MOE_FFN_INVALID_ARG = -1,        /* NULL pointer, bad shape, aliasing, N out of range */
  MOE_FFN_UNSUPPORTED = -2,        /* a shape outside the supported set */
  MOE_FFN_WORKSPACE_TOO_SMALL = -3,/* ws_bytes below moe_ffn_workspace_size(n_tokens) */
  MOE_FFN_OUT_OF_MEMORY = -4,      /* device allocation failed (weights create) */
  MOE_FFN_HIP_ERROR = -5,          /* a HIP runtime call or launch failed */
  MOE_FFN_SCRATCH_TOO_SMALL = -6   /* moe_ffn_prefill_static: the batch needs more
                                      than MOE_FFN_STATIC_SCRATCH_BYTES of workspace */
} moe_ffn_status;

/* Layer shape.  norm_topk_prob: #408 "Hypothesis" names it; OLMoE uses 0. */
typedef struct moe_ffn_dims {
  int32_t d_model;        /* hidden size d */
  int32_t n_experts;      /* routed experts E */
  int32_t top_k;          /* active experts per token (na) */
  int32_t d_ffn;          /* routed expert intermediate size F */
  int32_t d_shared_ffn;   /* shared expert intermediate size, 0 = no shared expert */
  int32_t norm_topk_prob; /* 1: renormalise the k selected softmax weights */
} moe_ffn_dims;

/* Opaque, library-owned device copy of one layer's weights in the layout the
 * kernels read (int8 code planes in MFMA operand order plus binary16 scale
 * planes; the router matrix transposed). */
typedef struct moe_ffn_weights moe_ffn_weights;

/* Optional caller-owned device buffers that receive the routing decisions and
 * intermediate products of a call (for parity checks).  Any member may be
 * NULL.  Shapes: topk_ids / topk_w [N][k]; shared_gate [N]; exp_start
 * [E+1(+1 with a shared expert)]; exp_tok_i / exp_tok_k [N*k (+N)]; xq [N][d]
 * int8 (16-byte aligned, else MOE_FFN_INVALID_ARG); xs [N][d/32] binary16
 * bits; partial [N][k(+1)][d] fp32 unweighted expert outputs, slot k holding
 * the shared expert.  They must not overlap the inputs, `out` or the
 * workspace. */
typedef struct moe_ffn_routing {
  int32_t* topk_ids;
  float* topk_w;
  float* shared_gate;
  int32_t* exp_start;
  int32_t* exp_tok_i;
  int32_t* exp_tok_k;
  int8_t* xq;
  uint16_t* xs;
  float* partial;
} moe_ffn_routing;

/* Build a weights handle (load time; #388 "Measurement discipline": one-time
 * setup belongs at load, not in the timed path).
 *   router_w     fp32 [E][d] row-major.
 *   router_bias  fp32 [E], or NULL for no bias (added to the logits before
 *                both the top-k and the softmax).
 *   gate_q8, up_q8   Q8_0 [E][F][d/32] blocks of 34 bytes {binary16 scale,
 *                int8 q[32]}, rows contiguous, unpadded (#406 "References":
 *                Q8_0 MMQ).
 *   down_q8      Q8_0 [E][d][F/32] blocks.
 *   sh_gate_q8, sh_up_q8 [Fs][d/32], sh_down_q8 [d][Fs/32], sh_gate_vec fp32
 *                [d]: the shared expert and its gate; all NULL when
 *                d_shared_ffn == 0, all non-NULL otherwise.
 * The inputs are read on `stream`; the call synchronises `stream` before it
 * returns, after which the caller may free them.  On success *out owns
 * device memory released by moe_ffn_weights_destroy. */
int moe_ffn_weights_create(const moe_ffn_dims* dims, const float* router_w,
                           const float* router_bias, const void* gate_q8, const void* up_q8,
                           const void* down_q8, const void* sh_gate_q8, const void* sh_up_q8,
                           const void* sh_down_q8, const float* sh_gate_vec, hipStream_t stream,
                           moe_ffn_weights** out);

/* Expert weight formats of moe_ffn_weights_create_fmt. */
#define MOE_FFN_FMT_Q8_0 0 /* 34-byte blocks of 32 {binary16 scale, int8 q[32]} */
#define MOE_FFN_FMT_Q4_K 1 /* 144-byte super-blocks of 256, see below */
#define MOE_FFN_FMT_Q3_K 2 /* 110-byte super-blocks of 256, see below */

/* moe_ffn_weights_create with the expert rows (routed and shared, gate, up
 * and down) in `format`.  MOE_FFN_FMT_Q8_0 is moe_ffn_weights_create.
 * MOE_FFN_FMT_Q4_K (#406 "References" names Q4_K beside Q8_0 among the
 * formats of the int8 MMQ path): each row of n values is n/256 super-blocks
 * of 144 bytes {binary16 d, binary16 dmin, 12 bytes of 6-bit sub-block
 * scales sc_j and mins m_j, 128 bytes of 4-bit codes}, the k-quant
 * super-block: weight i of sub-block j (32 values) is
 * d * sc_j * q_i - dmin * m_j; sub-blocks 0-3 keep sc_j and m_j in the low 6
 * bits of bytes j and j+4, sub-blocks 4-7 take the low (sc) or high (m)
 * nibble of byte j+4 as the low 4 bits and the top 2 bits of byte j-4 (sc)
 * or byte j (m) as the high 2; code i of sub-block j is the low (j even) or
 * high (j odd) nibble of code byte 32*(j/2)+i.  Layouts: gate/up [E][F][d/256]
 * super-blocks, down [E][d][F/256], shared [Fs][d/256] and [d][Fs/256].
 * The expert products are then the int8 activation blocks dotted with the
 * dequantised rows, per 32-block sa * (d * sc * C - dmin * m * A) with C the
 * int32 code dot product and A the sum of the activation codes, summed in
 * fp32.  Q4_K needs d_model, d_ffn and d_shared_ffn to be multiples of 256
 * (else MOE_FFN_UNSUPPORTED), and rejects with MOE_FFN_UNSUPPORTED weights
 * whose d * sc or dmin * m overflows binary16.  A Q4_K handle serves every
 * prefill entry point and moe_ffn_decode (which then runs the prefill
 * launches); moe_ffn_dbg_block_sums returns MOE_FFN_UNSUPPORTED for it.
 * MOE_FFN_FMT_Q3_K (the format of the Q3_K expert GEMM of #388 "Key
 * references"): each row of n values is n/256 super-blocks of 110 bytes {32
 * bytes of high bits, 64 bytes of 2-bit codes, 12 bytes of 6-bit sub-block
 * scales, binary16 d}, the 3-bit k-quant super-block: weight 128h+32g+l has
 * the 2-bit code (code byte 32h+l >> 2g) & 3 and the high bit (high-bit byte
 * l >> 4h+g) & 1, q = code - 4 when that bit is clear; it lies in 16-value
 * sub-block s = 8h+2g+l/16, whose scale sc_s takes nibble s/8 (low first) of
 * scale byte s%8 as its low 4 bits and bits 2(s/4)..2(s/4)+1 of scale byte
 * 8+s%4 as its high 2; the weight is d * (sc_s - 32) * q.  Layouts as for
 * Q4_K with 110-byte super-blocks; d_model, d_ffn and d_shared_ffn multiples
 * of 256.  The library expands Q3_K rows at load into int8 blocks holding the
 * same values exactly (per 32 values the scale -d and the codes
 * -(sc_s - 32) * q, which lie in [-128, 124]), so a Q3_K handle serves every
 * entry point, decode and the block-sum dump included (the dump's sums are
 * those of the expanded codes), with the Q8_0 planes' memory footprint.
 * The expansion needs a temporary device buffer of 34/32 bytes per weight
 * during the call.  Any other format is MOE_FFN_INVALID_ARG.  The other
 * arguments and the ownership rules are those of moe_ffn_weights_create. */
int moe_ffn_weights_create_fmt(const moe_ffn_dims* dims, int32_t format, const float* router_w,
                               const float* router_bias, const void* gate, const void* up,
                               const void* down, const void* sh_gate, const void* sh_up,
                               const void* sh_down, const float* sh_gate_vec, hipStream_t stream,
                               moe_ffn_weights** out);

/* Release a handle (NULL is accepted).  The caller must ensure no enqueued
 * work still reads it. */
int moe_ffn_weights_destroy(moe_ffn_weights* w);

/* Host-side query: the dims a handle was built with. */
int moe_ffn_weights_dims(const moe_ffn_weights* w, moe_ffn_dims* dims_out);

/* Workspace bytes needed by a prefill or decode call over up to max_tokens
 * tokens (host-side query, nothing enqueued).  The size never decreases as
 * max_tokens grows, so a workspace sized once for max_tokens serves every
 * prefill or decode call with n_tokens <= max_tokens. */
int moe_ffn_workspace_size(const moe_ffn_weights* w, int32_t max_tokens, size_t* bytes);

/* The same size from the layer shape alone, before any weights exist (pure
 * host computation; no device call).  Returns the moe_ffn_weights_create
 * status for dims it would reject. */
int moe_ffn_workspace_size_for_dims(const moe_ffn_dims* dims, int32_t max_tokens, size_t* bytes);

/* The batched MoE FFN over n_tokens tokens (#406 "The work" item 2):
 * router + top-k + weights (+ shared gate), per-32 int8 quantiser, CSR
 * bucketing, one grouped gate/up + SwiGLU int8 GEMM launch over all experts
 * (and the shared expert), one grouped down GEMM launch, and the ordered
 * combine (#129 "Scope").
 *   x        fp32 [n_tokens][d], not modified.
 *   out      fp32 [n_tokens][d]; must not overlap x or the workspace.
 *   ws       device workspace of ws_bytes >= moe_ffn_workspace_size(n_tokens),
 *            256-byte aligned; contents on entry are ignored.
 *   routing  NULL, or optional outputs (see moe_ffn_routing).
 * Returns without a host synchronisation. */
int moe_ffn_prefill(const moe_ffn_weights* w, const float* x, int32_t n_tokens, float* out,
                    void* ws, size_t ws_bytes, const moe_ffn_routing* routing,
                    hipStream_t stream);

/* The layer in a residual stack (#388 "Why 676 needs a per-layer rewrite":
 * the residual stream runs through the layers one after another; the
 * combine + residual + RMSNorm fusion of the stack).  Computes the layer's
 * output y exactly as moe_ffn_prefill does, but never stores it: its combine
 * adds y to the residual stream and normalises the result,
 *   h  <- h + y                        (fp32 [n_tokens][d], in place)
 *   xn <- h / sqrt(mean(h^2) + eps)    (fp32 [n_tokens][d], unit gain),
 * with the same arithmetic, bit for bit, as moe_ffn_prefill followed by
 * moe_ffn_residual_rmsnorm(h, y, xn) on 16-byte aligned rows.  h and xn are
 * 16-byte aligned.  xn may be x itself (the next layer's input written over
 * this one's); otherwise xn, h, x and the workspace must not overlap.
 * eps >= 0.  The other arguments are those of moe_ffn_prefill.
 * Returns without a host synchronisation. */
int moe_ffn_prefill_residual(const moe_ffn_weights* w, const float* x, int32_t n_tokens, float* h,
                             float* xn, float eps, void* ws, size_t ws_bytes,
                             const moe_ffn_routing* routing, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation and results as moe_ffn_prefill, with the workspace taken from a
 * static device array of MOE_FFN_STATIC_SCRATCH_BYTES inside the library
 * instead of a caller buffer.  The call allocates nothing.  Every GPU the
 * library runs on holds its own copy of the array until the process ends;
 * all calls on one GPU share it, so calls that overlap in time on one GPU
 * (other streams, other threads) race and must be serialised by the caller.
 * A batch whose workspace (moe_ffn_workspace_size(n_tokens)) exceeds the
 * array returns MOE_FFN_SCRATCH_TOO_SMALL before anything is enqueued: at
 * the OLMoE-shaped layer (d 2048, 64 experts, top-8, ffn 1024) that is above
 * 2026 tokens, at the 35B-A3B-shaped layer (256 experts, top-8, ffn 512 +
 * shared 512) above 1748.  x, out, routing and stream are those of
 * moe_ffn_prefill. */
#define MOE_FFN_STATIC_SCRATCH_BYTES (160u << 20)
int moe_ffn_prefill_static(const moe_ffn_weights* w, const float* x, int32_t n_tokens, float* out,
                           const moe_ffn_routing* routing, hipStream_t stream);

/* Chunked prefill (#388, second comment, "Prefill chunking": a long prompt
 * processed as consecutive micro-batches of a fixed size, 512 by default in
 * the pages' engines; the pages' idea is to upload each layer's experts once
 * per prompt across chunks).  Here every expert stays resident in HBM, and
 * what consecutive chunks can share is the GPU's 256 MB last-level cache
 * (MALL): the call runs moe_ffn_prefill over tokens [c0, c0 + chunk_tokens)
 * for c0 = 0, chunk_tokens, ... (the last chunk may be shorter), one after
 * another on `stream`, reusing one workspace.  With flags &
 * MOE_FFN_CHUNK_SERPENTINE, every second chunk walks its grouped GEMMs' tile
 * table from the last tile (experts in descending order), so that each chunk
 * starts on the experts whose weights the previous one streamed last.
 * Each token's routing and output are those of its own chunk's call, which
 * routes every token exactly as an unchunked call does (token-separable
 * routing); outputs agree with moe_ffn_prefill's to the fp32 output bar
 * (accumulation order inside a grouped GEMM tile depends on how many rows
 * share the tile).  ws_bytes >= moe_ffn_workspace_size(min(chunk_tokens,
 * n_tokens)).  x and out as for moe_ffn_prefill (whole batch); chunk_tokens
 * >= 1; unknown flag bits are MOE_FFN_INVALID_ARG.  Every check is made
 * before the first chunk is enqueued. */
#define MOE_FFN_CHUNK_SERPENTINE 1
int moe_ffn_prefill_chunked(const moe_ffn_weights* w, const float* x, int32_t n_tokens,
                            int32_t chunk_tokens, int32_t flags, float* out, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/* moe_ffn_prefill with stage timing (#388 "Measurement discipline": per-phase
 * timing buckets measured warm, with setup excluded).  stage_events points to
 * MOE_FFN_N_STAGE_EVENTS caller-created hipEvent_t handles (host array); event
 * i is recorded on `stream` before stage i and the last one after the final
 * stage, so hipEventElapsedTime(ev[i], ev[i+1]) is the device time of stage i:
 * 0 router logits, 1 top-k routing, 2 bucketing + activation quantiser,
 * 3 grouped gate/up + SwiGLU, 4 grouped down, 5 combine.  Same arguments and results as
 * moe_ffn_prefill otherwise. */
#define MOE_FFN_N_STAGE_EVENTS 7
int moe_ffn_prefill_profiled(const moe_ffn_weights* w, const float* x, int32_t n_tokens, float* out,
                             void* ws, size_t ws_bytes, const moe_ffn_routing* routing,
                             hipStream_t stream, hipEvent_t* stage_events);

/* Decode / small batch (#408 "Hypothesis" lever 1): the same computation for
 * 1 <= n_tokens <= 8, with the expert FFN run by one gathered launch per
 * stage in which each selected expert's weights are read once for all the
 * tokens that picked it.  Returns MOE_FFN_INVALID_ARG for n_tokens outside
 * [1, 8].  For Q4_K weights (whose planes the gathered matvecs do not read)
 * the call runs the prefill launches instead, with the same results contract. */
int moe_ffn_decode(const moe_ffn_weights* w, const float* x, int32_t n_tokens, float* out,
                   void* ws, size_t ws_bytes, const moe_ffn_routing* routing,
                   hipStream_t stream);

/* moe_ffn_decode with stage timing (#388 "Measurement discipline"), like
 * moe_ffn_prefill_profiled: stage_events points to MOE_FFN_N_DECODE_STAGE_EVENTS
 * caller-created hipEvent_t handles; event i is recorded on `stream` before
 * decode stage i and the last one after the final stage: 0 router logits +
 * activation quantiser, 1 routing + gathered gate/up matvec + SwiGLU, 2
 * gathered down matvec, 3 combine (for one token with at most 9 slots, k
 * plus the shared expert, stage 2 runs the down matvec and the combine in
 * one launch and stage 3 is empty).  Same arguments and results as
 * moe_ffn_decode otherwise. */
#define MOE_FFN_N_DECODE_STAGE_EVENTS 5
int moe_ffn_decode_profiled(const moe_ffn_weights* w, const float* x, int32_t n_tokens, float* out,
                            void* ws, size_t ws_bytes, const moe_ffn_routing* routing,
                            hipStream_t stream, hipEvent_t* stage_events);

/* Stage entry point: the ordered weighted combine on its own (#129 "Scope").
 * partial fp32 [n][kk][d] (kk = k, or k+1 when shared_gate != NULL, slot k
 * being the shared row), topk_w fp32 [n][k], shared_gate fp32 [n] or NULL,
 * out fp32 [n][d] (must not overlap the inputs).  1 <= k <= 16. */
int moe_ffn_combine(const float* partial, const float* topk_w, const float* shared_gate,
                    int32_t n, int32_t k, int32_t d, float* out, hipStream_t stream);

/* Stage entry point: the per-32-block int8 activation quantiser on its own.
 * v fp32 [n_values] (n_values % 32 == 0), q int8 [n_values], scales
 * binary16 bits [n_values/32]. */
int moe_ffn_quantize(const float* v, int64_t n_values, int8_t* q, uint16_t* scales,
                     hipStream_t stream);

/* Layer-stack helper (residual + RMSNorm between MoE layers; #388 "Why 676
 * needs a per-layer rewrite": the residual stream is sequential across
 * layers).  h fp32 [n][d] is updated in place to h + y when y != NULL (y
 * fp32 [n][d]); then xn fp32 [n][d] receives h / sqrt(mean(h^2) + eps)
 * (unit gain).  xn must not overlap h or y.  When d % 4 == 0 and h, y, xn
 * are 16-byte aligned, the sum of squares is taken in the order of
 * moe_ffn_prefill_residual's fused combine (4-column chunks per thread). */
int moe_ffn_residual_rmsnorm(float* h, const float* y, float* xn, int32_t n, int32_t d,
                             float eps, hipStream_t stream);

/* Parity hook: the integer core of a grouped GEMM (#406 "References": Q8_0
 * MMQ -- the products are exact int32 sums per 32-block before any scale).
 * Runs k-block `kblock` of 128-row tile `tile` against column strip `strip`
 * of the gate/up GEMM (gemm = 0; A = the tile's int8 activation rows, strip s
 * = gate rows 64s..64s+63 then up rows 64s..64s+63) or of the down GEMM
 * (gemm = 1; A = the tile's int8 h rows, strip s = down rows 128s..128s+127),
 * through the same copies, LDS layout, operand reads and int8 MFMA as the
 * product kernels, and writes
 *   sums     int32 [128][128]: sums[r][c] = sum over the block's 32 codes of
 *            A row r times weight row c of the strip (exact integers);
 *   a_codes  int8 [128][32] (16-byte aligned): the 32 codes A row r held;
 *   info     int32 [4]: {group, first CSR row, end CSR row, tile count}.
 *            Tile row r is CSR row first + r, valid while it is below end
 *            (rows past it hold no pair).  group is -1 when `tile` is at or
 *            past the tile count, -3 when strip or k-block lies outside that
 *            group's planes (nothing else is written then).
 * ws must hold the workspace of a moe_ffn_prefill (or _residual) call over
 * n_tokens tokens enqueued earlier on `stream`, and is not modified.  All
 * buffers are device memory; none may overlap the workspace.  Returns
 * MOE_FFN_INVALID_ARG for a tile at or past the workspace's tile bound, or a
 * strip or k-block outside every group's planes. */
int moe_ffn_dbg_block_sums(const moe_ffn_weights* w, void* ws, size_t ws_bytes, int32_t n_tokens,
                           int32_t gemm, int32_t tile, int32_t strip, int32_t kblock, int32_t* sums,
                           int8_t* a_codes, int32_t* info, hipStream_t stream);

/* Human-readable name of a status code (static storage). */
const char* moe_ffn_status_str(int status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_FFN_H */
