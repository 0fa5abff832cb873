/*
 * moe.h -- C ABI of a single-GPU sparse Mixture-of-Experts FFN layer (forward
 * pass, and its backward for training) for AMD Instinct MI355X (gfx950).
 *
 * The layer, as the pages describing it define it:
 *   [L] "Mixture of Experts (MoE)", AI Engineering from Scratch, Phase 07
 *       lesson 11: "Concept / FFN swap" (h + sum over the k chosen experts of
 *       gate * expert(h)), "The load balance problem" (aux loss, capacity,
 *       DeepSeek-V3 bias on selection only, +-gamma after each step),
 *       "Shared experts", "Build it / Step 1: the router".
 *   [N] "MoE architecture: load balancing and gating implementation"
 *       (nextadmin.net): "Load balancing" items 1-3 (C * N / E capacity).
 *   [G] "Mixture of Experts (MoE)" glossary (ultralytics.com): "How an MoE
 *       layer works", "Load balancing and expert capacity".
 *   [X] "Expert Parallelism for MoE Serving" (aiunderstanding.org):
 *       "Deep dive", "Technical insight" (dispatch by expert, capacity),
 *       "Future of expert parallelism for MoE serving" (fused dispatch and
 *       compute kernels, grouped GEMMs over many experts).
 *   [S] "How sparse models scale" (ircnf.com): quantised weights as the
 *       remedy for the memory size of large MoE models.
 *
 * Conventions shared by every entry point
 *   - Every pointer argument except `cfg` (and the struct pointers of
 *     moe_forward) is a DEVICE pointer on the current HIP device, allocated by
 *     the caller.  The library allocates, frees and synchronises nothing; all
 *     work is enqueued on `stream` and the call returns at once.
 *   - Device scalars (drop_count, aux) stay on the device.
 *   - Host-side validation runs before any launch.  On any non-MOE_OK status
 *     nothing has been enqueued, except MOE_ERR_HIP, which reports a failed
 *     launch (hipGetLastError) and may leave earlier kernels of the call queued.
 *   - Integer outputs are deterministic; floating-point outputs are
 *     bit-reproducible run to run (no floating-point atomics).
 *   - Storage types: MOE_BF16 stores x, weights, biases, intermediates and
 *     `out` as bfloat16 (bit patterns, uint16); MOE_F32 stores them as fp32.
 *     Router logits, gates and probability sums are always fp32;
 *     accumulation is always fp32.
 *   - Layouts are row-major.  Weights follow the [out, in] layout of a linear
 *     layer, so both GEMM operands are contiguous along the reduction axis:
 *       x [N, d]; w_router [E, d]; w1, w3 [E, F, d]; w2 [E, d, F];
 *       b1 [E, F]; b2 [E, d]; sh_w1, sh_w3 [Fs, d]; sh_w2 [d, Fs].
 *   - A slot is one (token, choice) pair; slot id s = t * k + j, where j
 *     orders the token's k experts by descending selection key.
 *   - Limits: 1 <= E <= 256; 1 <= k <= min(E, 16); for MOE_BF16, d and F (and
 *     Fs) must be multiples of 64 and device pointers 16-byte aligned.
 *     Anything else returns MOE_ERR_ARG or MOE_ERR_UNSUPPORTED.
 *   - The library is stateless; calls on different streams may run
 *     concurrently if their buffers are distinct.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_ARG = -1,          /* invalid size, NULL required pointer, NaN factor */
  MOE_ERR_UNSUPPORTED = -2,  /* dtype/activation combination or alignment not supported */
  MOE_ERR_WORKSPACE = -3,    /* ws_bytes smaller than moe_workspace_size() */
  MOE_ERR_HIP = -4,          /* a kernel launch failed */
  MOE_ERR_INTERNAL = -5
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef enum {
  /* [L] Step 1, [G]: key = z + sel_bias; gate = softmax over the k selected raw logits. */
  MOE_GATE_TOPK_SOFTMAX = 0,
  /* [L] DeepSeek-V3 approach, [N] item 3: p = softmax(z) over all E; key = p + sel_bias;
     gate = p of the selected experts renormalised to sum 1. */
  MOE_GATE_SOFTMAX_RENORM = 1,
  /* [G] Switch: argmax z (ties to the lower index); gate = p[argmax], not renormalised. */
  MOE_GATE_SWITCH_TOP1 = 2
} moe_gate_rule;

typedef enum {
  MOE_ACT_SWIGLU = 0,  /* [L] "FFN swap": (SiLU(x W1^T) * (x W3^T)) W2^T, no biases */
  MOE_ACT_GELU = 1     /* [G] example: GELU(x W1^T + b1) W2^T + b2, exact erf GELU */
} moe_act;

/* Where the kept rows of each expert live ([X] "Technical insight": per-expert
 * buffers, padded or dropped to a uniform shape).  PACKED: back to back,
 * offsets = exclusive scan of kept counts, N k rows at most.  PADDED: expert e
 * owns rows [e C, (e+1) C) (needs a finite capacity), kept rows first, padding
 * rows have perm = -1 and read as zero; every expert segment has C rows. */
typedef enum { MOE_CAPACITY_PACKED = 0, MOE_CAPACITY_PADDED = 1 } moe_capacity_layout;

/* Which slots an over-full expert keeps.  SLOT: the first C in slot order
 * s = t k + j.  CHOICE: the first C in (j, t) order - every token's first
 * choice before any second choice.  Rows of an expert follow the same order. */
typedef enum { MOE_PRIORITY_SLOT = 0, MOE_PRIORITY_CHOICE = 1 } moe_capacity_priority;

typedef struct moe_config {
  int64_t n_tokens;        /* N >= 0 */
  int32_t d_model;         /* d > 0 */
  int32_t n_experts;       /* E */
  int32_t top_k;           /* k */
  int32_t d_ff;            /* F: routed expert width */
  int32_t d_ff_shared;     /* Fs: always-on shared SwiGLU expert width; 0 = none ([L] "Shared experts") */
  int32_t act;             /* moe_act */
  int32_t ffn_bias;        /* 1: expert linears carry biases (MOE_ACT_GELU only) */
  int32_t gate_rule;       /* moe_gate_rule */
  float   capacity_factor; /* <= 0: unlimited; else C = floor(cf * N / E) ([N] item 2) */
  int32_t dtype;           /* moe_dtype */
  int32_t add_residual;    /* 1: out = x + MoE(x) ([L] "FFN swap": h + ...) */
  int32_t capacity_layout; /* moe_capacity_layout */
  int32_t capacity_priority; /* moe_capacity_priority */
} moe_config;

/* Rows R of the expert-ordered buffers (perm, x_perm, h_tmp, y_perm, and
 * pre_act's planes): N k for MOE_CAPACITY_PACKED, E C for MOE_CAPACITY_PADDED
 * with C = floor(cf * N / E) ([N] item 2), the capacity evaluated as the
 * library evaluates it (the factor's fp32 value times N over E in double,
 * truncated).  `capacity` (may be NULL) receives C, or INT32_MAX when the
 * capacity is unlimited.  Host only, launches nothing.  Errors: MOE_ERR_ARG
 * for an invalid config or a NULL `rows`. */
moe_status moe_expert_rows(const moe_config* cfg, int64_t* rows, int32_t* capacity);

/* Bytes of scratch that moe_forward needs for `cfg` (the step entry points
 * need at most this much too).  Host only, launches nothing. */
moe_status moe_workspace_size(const moe_config* cfg, size_t* bytes);

/* Router: logits, top-k selection and gates ([L] Step 1; [G] "How an MoE layer works").
 *   x          [N, d]     layer input (normalised hidden state)
 *   w_router   [E, d]     router weight (bias-free linear layer)
 *   logit_bias [E] fp32 | NULL   fixed offset added to every token's logits
 *   sel_bias   [E] fp32 | NULL   selection-only bias ([L] DeepSeek-V3 approach); never enters a gate
 *   logits_in  [N, E] fp32 | NULL  if given, used as the logits (the GEMM is skipped)
 *   logits     [N, E] fp32   out: z = x W_r^T + logit_bias (required when N > 0 unless logits_in is
 *              given; with logits_in it may be NULL, else receives a copy)
 *   topk_idx   [N, k] int32  out: chosen experts, descending key, exact ties to the lower index
 *   gates      [N, k] fp32   out: gate weights by `gate_rule`
 *   probsum    [E] fp32 | NULL   out: sum over tokens of softmax(z)[t, e] (for moe_aux_loss)
 *   ws/ws_bytes workspace of moe_workspace_size(cfg) bytes; required when probsum is
 *              requested.  bf16 routers with E <= 64 run one fused kernel (router GEMM,
 *              softmax, top-k and gates; the logits are still written).  Wider bf16
 *              routers with E a multiple of 64 compute the logits on the grouped-GEMM
 *              kernel with its K-split scratch when the workspace is given (for E in
 *              (128, 256] the top-k kernel completes the K-split logits); otherwise a
 *              dedicated router kernel runs.  All accumulate in fp32; their rounding
 *              orders differ.
 * Selection keys are formed and compared in fp64 from the fp32 logits and bias. */
moe_status moe_route(const moe_config* cfg, const void* x, const void* w_router,
                     const float* logit_bias, const float* sel_bias, const float* logits_in,
                     float* logits, int32_t* topk_idx, float* gates, float* probsum,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/* Dispatch: expert histogram, prefix scan, stable permutation, capacity and
 * the gather of token rows into expert order ([G] example's per-expert token
 * lists; [X] "Technical insight"; [N] item 2).
 *   topk_idx  [N, k] int32     from moe_route
 *   x         [N, d] | NULL    rows to gather (may be NULL when x_perm is NULL)
 *   counts    [E] int32        out: slots per expert before dropping (sum = N k)
 *   offsets   [E+1] int32      out: start row of each expert's segment: exclusive scan of
 *                              kept counts min(counts, C) (packed) or e C (padded)
 *   perm      [R] int32        out: perm[p] = slot id at expert-sorted position p
 *                              (p < offsets[E]), in priority order within an expert;
 *                              -1 on padding rows (R = N k packed, E C padded)
 *   slot_pos  [N k] int32      out: position of slot s in perm, -1 if dropped
 *   drop_count int64 | NULL    out: sum_e max(0, counts_e - C)
 *   x_perm    [R, d] | NULL    out: x_perm[p] = x[perm[p] / k] for p < offsets[E] (zero rows
 *                              where perm[p] = -1);
 *                              NULL skips the row copy (moe_expert_up_gather then
 *                              reads the token rows through perm)
 * Each expert keeps its first C slots in the order cfg->capacity_priority
 * names (ascending slot id by default). */
moe_status moe_permute(const moe_config* cfg, const int32_t* topk_idx, const void* x,
                       int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* slot_pos,
                       int64_t* drop_count, void* x_perm, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/* moe_permute for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same arguments
 * and results (bit-identical), but no workspace.  Its scratch (per-slot ranks
 * and per-block expert counts, 5 MiB) is a static device array inside the
 * library, one copy per GPU, held until the process ends; the call allocates
 * and frees nothing.  Limit: N k <= 2^20 slots (E <= 256 as everywhere);
 * larger batches return MOE_ERR_WORKSPACE before any launch.  Every call on a
 * GPU shares that GPU's scratch: calls that overlap on one GPU (different
 * streams, or host threads) race and must be serialised by the caller.
 * Errors as moe_permute, plus MOE_ERR_HIP if the scratch address cannot be
 * obtained on the current device. */
moe_status moe_permute_noalloc(const moe_config* cfg, const int32_t* topk_idx, const void* x,
                               int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* slot_pos,
                               int64_t* drop_count, void* x_perm, hipStream_t stream);

/* Grouped expert FFN over the ragged expert segments of x_perm ([L] "FFN swap";
 * [X] "Future of expert parallelism": grouped GEMMs that batch many experts).  Rows
 * [offsets[e], offsets[e+1]) of x_perm go through expert e.
 *   w3 must be NULL for MOE_ACT_GELU; b1, b2 are NULL unless cfg->ffn_bias.
 *   h_tmp  [R, F]  scratch/out: activated hidden rows (storage dtype)
 *   y_perm [R, d]  out: expert outputs in x_perm's row order (storage dtype)
 * Equivalent to moe_expert_up followed by moe_expert_down. */
moe_status moe_expert_ffn(const moe_config* cfg, const void* x_perm, const int32_t* offsets,
                          const void* w1, const void* w3, const void* w2,
                          const void* b1, const void* b2, void* h_tmp, void* y_perm,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/* First half of moe_expert_ffn: h = act(x_perm W1_e^T [, x_perm W3_e^T] [+ b1_e]). */
moe_status moe_expert_up(const moe_config* cfg, const void* x_perm, const int32_t* offsets,
                         const void* w1, const void* w3, const void* b1, void* h_tmp,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_expert_up with the dispatch gather fused into the GEMM's operand loads
 * ([X] "Future of expert parallelism": fused dispatch and compute kernels): row p of the expert order
 * is token row x[perm[p] / k], so no x_perm copy is made.
 *   x     [N, d]     token rows
 *   perm  [R] int32  from moe_permute
 * Results are bit-identical to moe_expert_up on the gathered x_perm.
 * MOE_ERR_UNSUPPORTED when a bf16 x exceeds 2 GiB - 1 MiB (the kernel's 32-bit
 * buffer offsets); moe_forward then falls back to the copy. */
moe_status moe_expert_up_gather(const moe_config* cfg, const void* x, const int32_t* perm,
                                const int32_t* offsets, const void* w1, const void* w3,
                                const void* b1, void* h_tmp, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/* moe_expert_up_gather that also keeps the pre-activations for moe_backward
 * (the training forward; [L] "The load balance problem" trains the layer):
 *   pre_act [n, R, F] bf16 out: plane 0 = x W1_e^T (+ b1_e for GELU), plane 1 =
 *   x W3_e^T (SwiGLU only; n = 2 for SwiGLU, 1 for GELU), rows in expert order,
 *   R = rows of the expert-ordered buffers.  Caller-owned device memory.
 * bf16 storage only (MOE_ERR_UNSUPPORTED otherwise); other arguments and errors
 * as moe_expert_up_gather; pre_act NULL is MOE_ERR_ARG when N > 0. */
moe_status moe_expert_up_save(const moe_config* cfg, const void* x, const int32_t* perm,
                              const int32_t* offsets, const void* w1, const void* w3,
                              const void* b1, void* h_tmp, void* pre_act, void* ws, size_t ws_bytes,
                              hipStream_t stream);

/* Second half of moe_expert_ffn: y = h W2_e^T [+ b2_e]. */
moe_status moe_expert_down(const moe_config* cfg, const void* h_tmp, const int32_t* offsets,
                           const void* w2, const void* b2, void* y_perm,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_expert_down with the combine fused into its epilogue, for top-1 routing
 * (top_k = 1; [X] "Future of expert parallelism": dispatch and combine fused into the expert
 * compute; [G] "Load balancing and expert capacity": a token over capacity
 * keeps the residual).  Each token has at most one slot, so the row holding
 * it is the token's only writer:
 *   out[t] = [residual_t] + [shared_y_t] + gates[t] * Y_row   (kept slot)
 *   out[t] = [residual_t] + [shared_y_t]                       (dropped)
 * with Y_row = h_row W2_e^T [+ b2_e] rounded to bf16 first, fp32 sums, one
 * rounding: bit-identical to moe_expert_down followed by moe_combine.
 *   perm [R], slot_pos [N], gates [N] from moe_route / moe_permute;
 *   residual, shared_y [N, d] or NULL; out [N, d].  No y_perm is written
 *   (moe_backward needs the unfused moe_expert_down).
 * Errors: MOE_ERR_UNSUPPORTED for top_k != 1, fp32 storage or a pointer not
 * 16-byte aligned; otherwise as moe_expert_down. */
moe_status moe_expert_down_combine(const moe_config* cfg, const void* h_tmp, const int32_t* offsets,
                                   const int32_t* perm, const int32_t* slot_pos, const float* gates,
                                   const void* w2, const void* b2, const void* residual,
                                   const void* shared_y, void* out, void* ws, size_t ws_bytes,
                                   hipStream_t stream);

/* fp8 weight-only experts ([S] "How sparse models scale": quantised weights are
 * how large MoE models fit in memory; the format here is OCP E4M3, round to
 * nearest).  Each row of a weight matrix stored [out, in] gets one fp32 scale:
 * scale = amax / 448 (1 for an all-zero row), code = nearest E4M3 value to
 * w * (448 / amax), ties to the even code, saturating at +-448.  The product
 * then uses w = value(code) * scale; activations stay bf16, accumulation fp32.
 *
 * moe_quantize_fp8: quantise a bf16 matrix w [rows, cols] (device) into codes
 *   q [rows, cols] uint8 and scales [rows] fp32 (both device, caller-owned).
 *   For cols % 4 == 0, w must be 16-byte and q 4-byte aligned.  Codes are a
 *   deterministic function of w (fp32 arithmetic with correctly rounded
 *   division).  Expert weights W1, W3 [E, F, d] are rows = E*F, cols = d;
 *   W2 [E, d, F] is rows = E*d, cols = F. */
moe_status moe_quantize_fp8(const void* w, int64_t rows, int32_t cols, uint8_t* q, float* scales,
                            hipStream_t stream);

/* moe_expert_up_gather with fp8 weights: h = act(x[perm] (W1q*s1)^T [, x[perm] (W3q*s3)^T] [+ b1]).
 *   w1q, w3q [E, F, d] uint8 codes, 16-byte aligned; s1, s3 [E, F] fp32 scales;
 *   w3q / s3 NULL for MOE_ACT_GELU.  bf16 storage only (else MOE_ERR_UNSUPPORTED).
 * Every segment runs on 64-row tiles: the kernel streams the codes (half the
 * bytes of bf16) and expands them to bf16 exactly before the bf16 MFMA. */
moe_status moe_expert_up_fp8(const moe_config* cfg, const void* x, const int32_t* perm,
                             const int32_t* offsets, const uint8_t* w1q, const uint8_t* w3q,
                             const float* s1, const float* s3, const void* b1, void* h_tmp,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_expert_down with fp8 weights: y = h (W2q*s2)^T [+ b2]; w2q [E, d, F] codes,
 * s2 [E, d] scales. */
moe_status moe_expert_down_fp8(const moe_config* cfg, const void* h_tmp, const int32_t* offsets,
                               const uint8_t* w2q, const float* s2, const void* b2, void* y_perm,
                               void* ws, size_t ws_bytes, hipStream_t stream);

/* Shared expert ([L] "Shared experts": every token passes through it, weight 1):
 * y_sh[N, d] = (SiLU(x sh_w1^T) * (x sh_w3^T)) sh_w2^T.  h_tmp is [N, Fs]. */
moe_status moe_shared_ffn(const moe_config* cfg, const void* x, const void* sh_w1,
                          const void* sh_w3, const void* sh_w2, void* h_tmp, void* y_sh,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/* Gate-weighted combine into token order ([L] "FFN swap"; [G] example):
 *   out[t] = [residual[t]] + [shared_y[t]] + sum_{j < k, slot_pos[t k + j] >= 0}
 *            gates[t, j] * y_perm[slot_pos[t k + j]],
 * summed in ascending j with fp32 accumulation.  A token whose slots were all
 * dropped receives exactly residual[t] (+ shared_y[t]) ([N] item 2; [G]).
 *   residual, shared_y: [N, d] or NULL; out [N, d] (storage dtype). */
moe_status moe_combine(const moe_config* cfg, const void* y_perm, const int32_t* slot_pos,
                       const float* gates, const void* residual, const void* shared_y,
                       void* out, hipStream_t stream);

/* Aux-loss-free balancing step ([L] "The load balance problem", DeepSeek-V3
 * approach; [L] Step 2): signs[e] = sign(counts[e] * E - N k) (int8: +1 over
 * target, -1 under, 0 on target; signs may be NULL); sel_bias[e] -= gamma *
 * signs[e] in fp32, in place.  Intended to run after the forward pass whose
 * counts it uses. */
moe_status moe_bias_update(const moe_config* cfg, const int32_t* counts, float gamma,
                           float* sel_bias, int8_t* signs, hipStream_t stream);

/* Auxiliary load-balance loss value ([G] "Load balancing and expert capacity";
 * [N] item 1): aux = E * sum_e (counts[e] / (N k)) * (probsum[e] / N), one
 * fp32 device scalar.  counts are pre-drop. */
moe_status moe_aux_loss(const moe_config* cfg, const int32_t* counts, const float* probsum,
                        float* aux, hipStream_t stream);

/* Device pointers of one layer's weights (NULL where the config has none). */
typedef struct moe_weights {
  const void*  w_router;     /* [E, d] */
  const float* logit_bias;   /* [E] fp32 | NULL */
  const void*  w1;           /* [E, F, d] */
  const void*  w3;           /* [E, F, d] (SwiGLU) */
  const void*  w2;           /* [E, d, F] */
  const void*  b1;           /* [E, F] (ffn_bias) */
  const void*  b2;           /* [E, d] (ffn_bias) */
  const void*  sh_w1;        /* [Fs, d] (d_ff_shared > 0) */
  const void*  sh_w3;        /* [Fs, d] */
  const void*  sh_w2;        /* [d, Fs] */
} moe_weights;

/* Device pointers of one layer's outputs.  `out` is required; every other
 * pointer may be NULL (the value is then kept in the workspace only). */
typedef struct moe_outputs {
  void*    out;              /* [N, d] storage dtype */
  float*   logits;           /* [N, E] */
  int32_t* topk_idx;         /* [N, k] */
  float*   gates;            /* [N, k] */
  int32_t* counts;           /* [E] pre-drop */
  int32_t* offsets;          /* [E+1] */
  int32_t* perm;             /* [R] */
  int32_t* slot_pos;         /* [N k] */
  int64_t* drop_count;       /* scalar */
  float*   probsum;          /* [E] */
  float*   aux;              /* scalar; computed when non-NULL */
  int8_t*  signs;            /* [E]; bias step runs when bias_gamma > 0 */
  float*   sel_bias_next;    /* [E] sel_bias - gamma * signs; may alias the sel_bias input */
  float    bias_gamma;       /* > 0: run the bias step after the forward pass (needs sel_bias
                                and sel_bias_next); 0 with signs != NULL: signs only */
} moe_outputs;

/* The whole layer: route -> permute -> grouped expert FFN -> [shared expert]
 * -> combine -> [aux loss] -> [bias step], all enqueued on `stream`.  The
 * up projection gathers the token rows itself (moe_expert_up_gather) when
 * the token matrix fits its 32-bit offsets; with top_k = 1 and bf16 storage
 * the combine runs in the down projection's epilogue
 * (moe_expert_down_combine).  Both are bit-identical to the unfused steps.
 *   x        [N, d]; residual [N, d] | NULL (NULL with add_residual = 1 uses x)
 *   sel_bias [E] fp32 | NULL (selection bias used by this pass) */
moe_status moe_forward(const moe_config* cfg, const moe_weights* w, const void* x,
                       const void* residual, const float* sel_bias, const moe_outputs* o,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ backward
 * Gradients of the layer for an upstream gradient `dout` of `out` and `d_aux`
 * of the auxiliary loss ([L] "The load balance problem": the aux loss is a
 * second gradient signal into the router; the bias step, moe_bias_update,
 * follows each training step).  The routing decisions (selection, capacity)
 * are taken as fixed: they are piecewise constant in the inputs.  Gradients
 * flow through the gate weights (rule A: softmax over the selected logits;
 * rule B: renormalised softmax probabilities; rule C: the argmax probability)
 * into the logits, the router weight, the logit bias and the input; through
 * the kept slots' expert FFNs (pre-activations recomputed); the shared expert;
 * and the residual.  bf16 storage only (MOE_ERR_UNSUPPORTED otherwise):
 * bf16 operands and intermediates, fp32 accumulation, fp32 weight gradients.
 */
typedef struct moe_saved {      /* forward state of the same call, as the step entry points return it */
  const float*   logits;        /* [N, E] fp32 */
  const int32_t* topk_idx;      /* [N, k] */
  const float*   gates;         /* [N, k] */
  const int32_t* counts;        /* [E] (used for the aux-loss gradient) */
  const int32_t* offsets;       /* [E+1] */
  const int32_t* perm;          /* [R] */
  const int32_t* slot_pos;      /* [N k] */
  const void*    y_perm;        /* [R, d] expert outputs (storage dtype) */
  const void*    pre_act;       /* [n, R, F] from moe_expert_up_save, or NULL: recomputed */
} moe_saved;

typedef struct moe_grads {      /* device outputs; fp32 unless noted */
  void*  dx;                    /* [N, d] storage dtype (required) */
  float* dw_router;             /* [E, d] | NULL */
  float* dlogit_bias;           /* [E] | NULL */
  float* dw1;                   /* [E, F, d] (required) */
  float* dw3;                   /* [E, F, d] (required for SwiGLU) */
  float* dw2;                   /* [E, d, F] (required) */
  float* db1;                   /* [E, F] (required with ffn_bias) */
  float* db2;                   /* [E, d] (required with ffn_bias) */
  float* dsh_w1;                /* [Fs, d] (required with a shared expert) */
  float* dsh_w3;                /* [Fs, d] */
  float* dsh_w2;                /* [d, Fs] */
  float* dgates;                /* [N, k] | NULL: dL/dgates */
} moe_grads;

/* Workspace bytes moe_backward needs: the forward's scratch (the backward's
 * tile lists, K-split partials), the pre-activations when the forward did not save them,
 * the expert-ordered token rows, the intermediate gradients (dY, dH, dA, dX,
 * dz) and the shared expert's intermediates.  No weight copies: every product
 * reads the weights in their stored layout.  Host only. */
moe_status moe_backward_workspace_size(const moe_config* cfg, size_t* bytes);

/* x [N, d], dout [N, d] (storage dtype), weights as for moe_forward; `saved`
 * holds the forward state of the same inputs (caller-owned device buffers,
 * read only).  d_aux multiplies the aux-loss gradient (pass 0 when the loss is
 * not used).  Every gradient is overwritten, not accumulated; unused experts
 * get zero weight gradients.  The call is deterministic (no atomics).
 * Errors, before any launch: MOE_ERR_ARG for a missing required pointer or a
 * NaN d_aux; MOE_ERR_UNSUPPORTED for fp32 storage, a pointer not 16-byte
 * aligned, or a token matrix beyond the 32-bit gather offsets; MOE_ERR_WORKSPACE
 * when ws_bytes is below moe_backward_workspace_size. */
moe_status moe_backward(const moe_config* cfg, const moe_weights* w, const void* x, const void* dout,
                        float d_aux, const moe_saved* saved, const moe_grads* grads, void* ws,
                        size_t ws_bytes, hipStream_t stream);

/* Measurement probes.  They compute nothing of the layer: they measure, on
 * the GPU at hand, the practical ceilings of the two resources its kernels are
 * bound by, so that a benchmark can state roofline fractions against what the
 * chip sustains as well as against its published peaks (HBM 8 TB/s, dense
 * bf16 MFMA 2.5 PFLOP/s).  Each enqueues one kernel on `stream`; time it with
 * events on that stream.
 *
 * moe_probe_hbm_read: reads `bytes` of the device buffer `buf` once (16-byte
 *   nontemporal loads, one persistent workgroup per CU, 256 KB chunks dealt
 *   round robin).  `sink` is a device uint32 the kernel may overwrite.
 *   Errors: MOE_ERR_ARG for a NULL buf or sink with bytes > 0;
 *   MOE_ERR_UNSUPPORTED when buf is not 16-byte aligned or bytes is not a
 *   multiple of 16.
 * moe_probe_mfma_bf16: every CU runs 8 wavefronts that each issue `iters`
 *   rounds of two independent v_mfma_f32_32x32x16_bf16 on operands read
 *   once from `operands` (at least 4 KB of device bf16 data, 16-byte aligned;
 *   random values give the switching activity of real data).  `sink` is a
 *   device float the kernel may overwrite.  Errors: MOE_ERR_ARG for iters < 0
 *   or a NULL pointer with iters > 0; MOE_ERR_UNSUPPORTED for an unaligned
 *   operand buffer.
 * moe_probe_mfma_flop_per_iter: the FLOPs one iteration of
 *   moe_probe_mfma_bf16 performs on the current device (host only). */
moe_status moe_probe_hbm_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);
moe_status moe_probe_mfma_bf16(const void* operands, int64_t iters, float* sink, hipStream_t stream);
moe_status moe_probe_mfma_flop_per_iter(int64_t* flop);

/* Static text for a status code. */
const char* moe_status_str(moe_status s);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
