/*
 * libmoe: one Mixture-of-Experts layer, forward and backward, on one AMD Instinct
 * MI355X (gfx950).  Plain C ABI: every tensor argument is a DEVICE pointer that the
 * caller allocated; sizes come from moe_config_t; `stream` is a hipStream_t (NULL =
 * the default stream).  The library allocates no memory, keeps no state between calls
 * (the only HIP objects it creates are the events of one moe_layer_bwd call given a second
 * stream, destroyed before that call returns) and never synchronises the host: every call
 * only enqueues kernels on `stream`.
 *
 * Deviation from the plain statement of the layer: y, dy and dx are fp32 in every layer,
 * also where the activations are bf16, because one bf16 rounding of the combined output
 * (or of the input gradient) costs up to 2e-2 of its RMS on its own.
 *
 * Sources, cited by page title and section:
 *   [HB] "The Ultimate MoE Training Handbook" (Hugging Face).
 *   [LC] LeCompute, "MoE training: cluster, routing, load balancing".
 *
 * Notation: T tokens, d model width, E routed experts, k experts per token, F expert
 * FFN width, Fs shared-expert width (0 = none), A = T*k routed rows.
 *
 * Layouts (all row-major, contiguous):
 *   x                     [T, d]      activation dtype (act_dtype)
 *   y, dy, dx             [T, d]      fp32
 *   Wg                    [E, d]      fp32        router weight ([HB] §3.4 Count and size)
 *   W13                   [E, 2F, d]  act dtype   fc1 of each expert, gate rows then up rows
 *   W2                    [E, d, F]   act dtype   fc2 of each expert
 *   W13s [2Fs, d], W2s [d, Fs]        act dtype   shared expert
 *   logits, dlogits       [T, E]      fp32
 *   idx [T, k] int32, w [T, k] fp32   slot j: j-th best expert (key descending, ties to the
 *                                     lower expert index) and its mixing weight
 *   counts [E] int32, offsets [E+1] int32, row_of [T, k] int32, token_of [A] int32
 *   x_perm                [A, d]      act dtype, rows grouped by expert ascending, and by
 *                                     token ascending inside an expert
 *   H [A, 2F] fp32, Act [A, F] act dtype   fc1 output (gate half, then up half), SwiGLU
 *   Y_perm [A, d], Y_s [T, d]         fp32 expert outputs (same row order as x_perm)
 *   dX_perm [A, d]                    fp32 per-row input gradients
 *   dW13, dW2, dW13s, dW2s            weight gradients, shaped like the weights, in wgrad_dtype
 *
 * fp8 experts (w_dtype == MOE_FP8_E4M3): W13 and W2 hold e4m3 codes (one byte each)
 * with one fp32 scale per 128 x 128 block; x_perm and Act hold e4m3 codes with one scale
 * per row per 128 columns (x_perm_scale, Act_scale); H and Y_perm stay fp32.  The pages
 * give no low-precision expert recipe; the one taken is documented at moe_quantize_fp8.
 *
 * Precision: every GEMM multiplies act-dtype operands (bf16 on the matrix cores) with
 * fp32 accumulation.  Only GEMM operands are stored in bf16 (x_perm, Act, dY_perm, dH);
 * everything that is summed or differentiated further (H, expert outputs, per-row input
 * gradients, y, dx, router weight gradients) stays fp32: one bf16 rounding of a value five
 * to six standard deviations out is already 2e-2 of the tensor's RMS.  The expert weight
 * gradients are stored in wgrad_dtype: fp32, or bf16 (each element rounded once, to
 * nearest even, from its fp32 accumulator), like the bf16 weights they belong to.
 *
 * Errors: every argument is checked on the host before anything is launched.  A call
 * that fails a check launches nothing and returns MOE_ERR_INVALID_ARG,
 * MOE_ERR_UNSUPPORTED or MOE_ERR_WORKSPACE; a failed launch returns MOE_ERR_HIP.
 * moe_last_error() gives the text of the last failure on the calling thread.
 * Numerical faults (non-finite inputs) are not detected.
 *
 * Determinism: no floating-point atomics; every reduction runs in a fixed order, so
 * repeated calls on the same inputs give bit-identical outputs.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_WORKSPACE = 3,
  MOE_ERR_HIP = 4
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype_t;

/* [HB] §3.1 Router scoring, Gating function: softmax, sigmoid, or the square root of
 * softplus, s = sqrt(log(1 + e^l)). */
typedef enum { MOE_SOFTMAX = 0, MOE_SIGMOID = 1, MOE_SQRTSOFTPLUS = 2 } moe_score_t;

/* stats[]: aux loss, MaxVio, number of empty experts, max count, router z-loss,
 * sequence-wise aux loss (each loss already multiplied by its coefficient). */
#define MOE_NSTATS 6

/* The experts' gated activation on H = [gate | up] ([HB] §3.4 Activation):
 *   MOE_GLU_SWIGLU  Act = silu(gate) * up;
 *   MOE_GLU_CLAMP   the hard clamp: gate clamped from above at c and up to [-c, c], then
 *                   SwiGLU (the gradient passes where the input lies inside the interval);
 *   MOE_GLU_SITU    SiTU-GLU: s tanh(gate / s) sigmoid(gate) * up', with
 *                   up' = s_l tanh(up / s_l) when s_l > 0, else up. */
typedef enum { MOE_GLU_SWIGLU = 0, MOE_GLU_CLAMP = 1, MOE_GLU_SITU = 2 } moe_glu_t;

/*
 * The layer's settings, mirroring the flags of [HB] §2.5 Your first MoE (number of
 * experts, expert FFN width, top-k), §3.1 (score function, routed scaling factor),
 * §3.3 Aux loss (coefficient) and §3.4 Shared experts (shared width), plus the
 * balancing losses of §3.1 Precision (z-loss) and §3.3 Scope (sequence-wise loss).
 * Rules checked by moe_validate:
 *   1 <= k <= min(E, 32), E <= 2048, T >= 1, T*k < 2^31, d % 64 == 0, F % 64 == 0,
 *   Fs % 64 == 0; bf16: F % 128 == 0 and Fs % 128 == 0;
 *   pre_softmax is 0 or 1 and only with softmax scores (UNSUPPORTED otherwise);
 *   softmax with k == 1 needs pre_softmax (UNSUPPORTED otherwise: [HB] §3.1 Output
 *   scale, a softmax over one selected logit gives the router no gradient);
 *   aux_coeff, z_coeff, seq_aux_coeff finite and >= 0; seq_aux_coeff > 0 needs
 *   seq_len >= 1 dividing T (INVALID_ARG otherwise) and T / seq_len <= 65535;
 *   num_groups != 0: 1 <= num_groups <= 64 dividing E, 1 <= group_topk <= min(num_groups, k),
 *   k / group_topk <= E / num_groups and group_topk * E / num_groups >= k; num_groups == 0
 *   needs group_topk == 0 (INVALID_ARG otherwise);
 *   shared_gate is 0 or 1, and 1 needs Fs > 0 (INVALID_ARG otherwise);
 *   glu_kind MOE_GLU_CLAMP needs glu_c finite > 0; MOE_GLU_SITU needs glu_c finite > 0 and
 *   glu_c_linear finite >= 0 (INVALID_ARG otherwise);
 *   w_dtype == MOE_FP8_E4M3 (fp8 experts, see moe_quantize_fp8) needs act_dtype == bf16,
 *   Fs == 0, d % 128 == 0 and F % 128 == 0 (UNSUPPORTED otherwise).
 */
typedef struct moe_config {
  int32_t T, d, E, k, F, Fs;
  int32_t score;          /* moe_score_t */
  int32_t pre_softmax;    /* softmax only: 1 = top-k of the full softmax, weights not renormalised */
  float routed_scaling;   /* multiplies the renormalised weights ([HB] §3.1 Output scale) */
  float aux_coeff;        /* Switch aux-loss coefficient ([HB] §3.3 Aux loss) */
  int32_t act_dtype;      /* moe_dtype_t of activations (and of expert weights when w_dtype == 0) */
  int32_t w_dtype;        /* 0: expert weights in act_dtype; MOE_FP8_E4M3: e4m3 codes + scales */
  float z_coeff;          /* router z-loss coefficient ([HB] §3.1 Precision); 0 = off */
  float seq_aux_coeff;    /* sequence-wise aux-loss coefficient ([HB] §3.3 Scope); 0 = off */
  int32_t seq_len;        /* S of the sequence-wise loss: tokens are ordered [S, B], token
                             t = s * B + b is position s of sequence b, B = T / S */
  int32_t wgrad_dtype;    /* moe_dtype_t of the expert weight gradients: MOE_F32 (0), or
                             MOE_BF16 with bf16 activations (INVALID_ARG / UNSUPPORTED otherwise) */
  int32_t glu_kind;       /* moe_glu_t: the experts' gated activation ([HB] §3.4 Activation) */
  float glu_c;            /* MOE_GLU_CLAMP: the limit c; MOE_GLU_SITU: the gate cap s */
  float glu_c_linear;     /* MOE_GLU_SITU: the up-half cap s_l (0 = no cap) */
  int32_t num_groups;     /* group-limited routing ([HB] §3.1): experts in num_groups groups of
                             consecutive indices, 0 = off */
  int32_t group_topk;     /* groups a token keeps: those with the largest sum of their best
                             k / group_topk selection keys (ties to the lower group) */
  int32_t shared_gate;    /* 1: the shared expert's output is scaled by sigma(x . Wsg)
                             ([HB] §3.4 Shared experts, the gated form); needs Fs > 0 */
} moe_config_t;

typedef struct moe_weights {
  const float* Wg;          /* [E, d] fp32 */
  const float* bg;          /* [E] fp32 additive logit bias, or NULL */
  const float* expert_bias; /* [E] fp32 selection-only bias (sigmoid only), or NULL */
  const void* W13;          /* [E, 2F, d] */
  const void* W2;           /* [E, d, F] */
  const void* W13s;         /* [2Fs, d], NULL when Fs == 0 */
  const void* W2s;          /* [d, Fs],  NULL when Fs == 0 */
  const float* W13_scale;   /* fp8 weights only: [E, 2F/128, d/128] fp32 block scales */
  const float* W2_scale;    /* fp8 weights only: [E, d/128, F/128] fp32 block scales */
  const float* Wsg;         /* [d] fp32 gate weight of the shared expert, when shared_gate */
} moe_weights_t;

/* Tensors the forward writes and the backward reads (all caller-owned). */
typedef struct moe_saved {
  float* logits;     /* [T, E] */
  int32_t* idx;      /* [T, k] */
  float* w;          /* [T, k] */
  int32_t* counts;   /* [E] */
  int32_t* offsets;  /* [E+1] */
  int32_t* row_of;   /* [T, k] */
  int32_t* token_of; /* [A] */
  void* x_perm;      /* [A, d], or NULL (bf16 activations): the grouped fc1 and its weight
                        gradient then read row token_of[r] of x in place of row r, and the
                        grouped copy is never made */
  void* H;           /* [A, 2F] fp32 */
  void* Act;         /* [A, F] */
  void* Y_perm;      /* [A, d] fp32 */
  void* H_s;         /* [T, 2Fs] fp32, or NULL when Fs == 0 */
  void* Act_s;       /* [T, Fs]  or NULL */
  void* Y_s;         /* [T, d]   fp32, or NULL */
  float* x_perm_scale; /* fp8 weights only: [A, d/128], the scales of x_perm's e4m3 rows
                          (NULL with x_perm: the fc1 then reads the token rows' codes and
                          scales, kept in the forward workspace, through token_of) */
  float* Act_scale;    /* fp8 weights only: [A, F/128], the scales of Act's e4m3 rows */
  int32_t* seq_counts; /* [B, E] tokens of sequence b routed to e; needed when seq_aux_coeff > 0 */
  float* gs;           /* [T] the shared expert's gate values, when shared_gate */
} moe_saved_t;

/* Gradients written by moe_layer_bwd.  accumulate = 0 overwrites them; accumulate = 1
 * adds this call's gradients into the values the buffers hold (gradient accumulation over
 * micro-batches): each element becomes old + new in fp32, with the fp32 sum of one call
 * formed exactly as when overwriting; a bf16 gradient is rounded once from
 * old + the fp32 accumulator.  An expert without rows leaves its gradients untouched
 * (overwriting writes exact zeros).  Any other accumulate value -> MOE_ERR_INVALID_ARG. */
typedef struct moe_grads {
  float* dWg;  /* [E, d] fp32 */
  float* dbg;  /* [E] fp32, or NULL */
  void* dW13;   /* [E, 2F, d] in wgrad_dtype; experts with no rows get exact zeros */
  void* dW2;    /* [E, d, F] */
  void* dW13s;  /* [2Fs, d] or NULL when Fs == 0 */
  void* dW2s;   /* [d, Fs]  or NULL */
  float* dWsg;  /* [d] fp32, when shared_gate */
  int32_t accumulate; /* 0: overwrite, 1: add into the buffers */
} moe_grads_t;

const char* moe_status_string(moe_status_t status);
const char* moe_last_error(void);

/* Checks the configuration rules listed at moe_config_t.  Host only. */
moe_status_t moe_validate(const moe_config_t* cfg);

/* Workspace bytes the forward (router, permute, layer forward) and backward calls need.
 * Host only.  One workspace of max(fwd, bwd) bytes serves every call.  On bf16 layers
 * whose skew-split chunk (see moe_grouped_wgrad) is below T, the backward bytes include
 * the split's plan and (ceil(A / chunk) + floor(A / chunk)) fp32 partials of N x K for
 * the larger of the two routed weight gradients (268 MB on the Qwen3-Next-shaped layer). */
moe_status_t moe_workspace_size(const moe_config_t* cfg, size_t* fwd_bytes, size_t* bwd_bytes);

/* Router logits = x Wg^T (+ bg), fp32 ([HB] §3.1 Router scoring, Precision: the router's
 * linear layer runs in fp32).  x act dtype [T, d]; logits [T, E].  With bf16 activations
 * and E % 16 == 0 it runs on the bf16 matrix cores through an exact three-way bf16 split
 * of Wg (every product exact, fp32 accumulation); otherwise as an fp32 FMA GEMM.
 * ws: the workspace of moe_workspace_size (scratch for the split and the partial sums). */
moe_status_t moe_gate_logits(const moe_config_t* cfg, const void* x, const float* Wg, const float* bg,
                             float* logits, void* ws, size_t ws_bytes, void* stream);

/* Top-k router ([HB] §3.1 Gating function and Output scale; §3.3 Aux loss, Scope):
 *   keys: softmax -> the logits (also with pre_softmax: the full softmax ranks as the
 *         logits do); sigmoid / sqrt(softplus) -> s(l) + expert_bias, evaluated in fp64;
 *   idx: top-k of the keys, ties to the lower expert index;
 *   w:   softmax over the k selected logits; with pre_softmax the full softmax at the
 *        selected experts; or s(l_S) / (sum + 1e-20) (k > 1), s(l_S) (k == 1); times
 *        routed_scaling;
 *   counts[e]: tokens routed to e;
 *   prob_sum[e] = sum_t q_te (NULL ok), q the aux probabilities: the full softmax, or the
 *        scores normalised over all E, s / (sum_e s + 1e-20);
 *   stats[MOE_NSTATS] (NULL ok): aux = aux_coeff * E * sum_e f_e P_e, MaxVio, empty
 *        experts, max count, z = z_coeff * mean_t logsumexp(l_t)^2, and the sequence-wise
 *        loss seq_aux_coeff * mean_b E sum_e f_be P_be over the B = T / seq_len sequences;
 *   seq_counts [B, E] (needed when seq_aux_coeff > 0, else ignored): per-sequence counts.
 *   expert_bias must be NULL for softmax. */
moe_status_t moe_router_topk(const moe_config_t* cfg, const float* logits, const float* expert_bias,
                             int32_t* idx, float* w, int32_t* counts, float* prob_sum, float* stats,
                             int32_t* seq_counts, void* ws, size_t ws_bytes, void* stream);

/* moe_router_topk for callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): the same call and kernels, with no
 * workspace argument.  Its scratch (the router's block partials) lives in a static device
 * array of 8 MiB inside the library -- one per GPU, held until the process ends -- whose
 * device address is looked up once per device on the first call there.  The call allocates
 * nothing.  Every kernel fully writes the scratch it reads, so no clearing is needed, but
 * all calls on one GPU share that array: calls that overlap on one GPU (concurrent host
 * threads, or different streams) race and must not be issued.  Errors: as moe_router_topk,
 * plus MOE_ERR_WORKSPACE when the configuration needs more than the 8 MiB (the router's
 * partials are about 8 * E * ceil(T / 64) bytes, more with the sequence-wise loss), and
 * MOE_ERR_HIP when the array's address cannot be taken. */
moe_status_t moe_router_topk_noalloc(const moe_config_t* cfg, const float* logits, const float* expert_bias,
                                     int32_t* idx, float* w, int32_t* counts, float* prob_sum, float* stats,
                                     int32_t* seq_counts, void* stream);

/* Loss-free balancing bias, one update ([HB] §3.3 Load balancing, Loss-free bias):
 *   direction_e = sign(sum(counts) - counts[e] * E)   (integers: exact),
 *   step_e = direction_e * rate;  centered != 0: step_e -= (rate * sum_e direction_e) / E;
 *   expert_bias[e] += step_e,
 * each operation one fp32 rounding in that order.  counts [E] int32 (for example the
 * router's counts, or their sum over the micro-batches of a step, below 2^31);
 * expert_bias [E] fp32, updated in place.  Errors: rate not finite -> INVALID_ARG. */
moe_status_t moe_expert_bias_update(const moe_config_t* cfg, const int32_t* counts, float rate, int32_t centered,
                                    float* expert_bias, void* stream);

/* Quantile balancing, one micro-batch ([HB] §3.3 Load balancing, Quantile): the selection
 * bias is solved for instead of stepped.  All in fp32 (the router precision):
 *   keys = scores - beta; per token the k + 1 largest keys, key descending, ties to the
 *   lower expert index: idx [T, k] gets the first k, alpha [T] the (k+1)-th key;
 *   beta_local (NULL: routing only) [E]: per expert the (T k / E + 1)-th largest of
 *   scores[:, e] - alpha over the T tokens, the value only the expert's target share of
 *   T k / E tokens lies above.
 * scores [T, E] fp32 are the router's scores (for example the softmax probabilities or the
 * sigmoid scores), beta [E] fp32 the current bias.  ws: the forward workspace.
 * Errors: k >= E; beta_local requested and T * k not a multiple of E -> INVALID_ARG. */
moe_status_t moe_router_quantile(const moe_config_t* cfg, const float* scores, const float* beta, int32_t* idx,
                                 float* alpha, float* beta_local, void* ws, size_t ws_bytes, void* stream);

/* The step update of the quantile bias ([HB] §3.3 Quantile, the EMA):
 *   beta = ema * beta + (1 - ema) * beta_local, then the mean over the E experts is
 *   subtracted (summed in fp64 in a fixed order).  beta_local: the step's solution (the
 *   average over its micro-batches is the caller's).  Errors: ema outside [0, 1] -> INVALID_ARG. */
moe_status_t moe_quantile_bias_update(const moe_config_t* cfg, const float* beta_local, float ema, float* beta,
                                      void* stream);

/* Dropless permutation ([LC] "Read the timeline before blaming the network": tokens are
 * grouped by expert before the expert matmuls): offsets = exclusive prefix of the
 * per-expert counts; row_of[t, j] = row of (t, j); token_of[row] = t;
 * x_perm[row_of[t, j]] = x[t].  Rows inside an expert follow token order.
 * x_perm NULL: only the grouping is computed (x may then be NULL too); the grouped GEMMs
 * take token_of in place of the copy.
 * idx must hold, for each token, k distinct expert ids in [0, E) (the router's output
 * does).  Ids outside [0, E) are clamped into it and a repeated id leaves rows of token_of
 * unwritten: the results are then unspecified, but no access leaves the buffers. */
moe_status_t moe_permute(const moe_config_t* cfg, const void* x, const int32_t* idx, int32_t* offsets,
                         int32_t* row_of, int32_t* token_of, void* x_perm, void* ws, size_t ws_bytes,
                         void* stream);

/* Grouped SwiGLU experts ([HB] §3.4 Count and size, Activation): for each expert e, on its
 * rows [offsets[e], offsets[e+1]):  H = X W13[e]^T, Act = silu(H[:, :F]) * H[:, F:],
 * Y_perm = Act W2[e]^T (fp32).  When Fs > 0 the shared expert runs the same on x (all T
 * rows) into H_s, Act_s, Y_s ([HB] §3.4 Shared experts).
 * X is x_perm [A, d] (token_of NULL), or, with token_of [A] given and x_perm NULL, row
 * token_of[r] of x [T, d] for row r (bf16 activations only): the same products, bit for
 * bit, without the grouped copy.  Errors: both or neither of x_perm and token_of ->
 * MOE_ERR_INVALID_ARG; token_of with fp32 activations -> MOE_ERR_UNSUPPORTED. */
moe_status_t moe_grouped_gemm_swiglu(const moe_config_t* cfg, const void* x_perm, const int32_t* token_of,
                                     const int32_t* offsets, const void* W13, const void* W2, const void* x,
                                     const void* W13s, const void* W2s, void* H, void* Act, void* Y_perm,
                                     void* H_s, void* Act_s, void* Y_s, void* ws, size_t ws_bytes, void* stream);

/* Weighted combine ([LC] "An expert transforms numbers inside the model": the weighted
 * sum of the selected outputs, coordinate by coordinate; [HB] §3.4 Shared experts: the
 * shared output is added at weight 1, or at its sigmoid gate gs[t]):
 *   y[t] = sum_j w[t, j] * Y_perm[row_of[t, j]] (+ gs[t] * Y_s[t]), fp32 accumulation, slot
 *   order.  gs [T] NULL means 1. */
moe_status_t moe_unpermute_combine(const moe_config_t* cfg, const float* Y_perm, const int32_t* row_of,
                                   const float* w, const float* Y_s, const float* gs, float* y, void* stream);

/* The shared expert's sigmoid gate ([HB] §3.4 Shared experts: output * sigmoid(x Wsg)):
 * gs[t] = sigma(<x[t], Wsg>), the dot in fp32.  x act dtype [T, d], Wsg [d] fp32 (16-byte
 * aligned), gs [T] fp32. */
moe_status_t moe_shared_gate(const moe_config_t* cfg, const void* x, const float* Wsg, float* gs, void* stream);

/* Its weight gradient: dWsg = sum_t dl_s[t] x[t] (dl_s from moe_unpermute_combine_bwd),
 * partial sums over 256-token chunks then over the chunks, in a fixed order.  ws: the
 * backward workspace. */
moe_status_t moe_shared_gate_bwd(const moe_config_t* cfg, const void* x, const float* dl_s, float* dWsg, void* ws,
                                 size_t ws_bytes, void* stream);

/* Whole forward: gate logits, router, permute, grouped experts (+ shared), combine.
 * Fills *saved for the backward.  stats as in moe_router_topk (NULL ok); saved->seq_counts
 * receives the per-sequence counts when seq_aux_coeff > 0.
 * fp8 experts: x (bf16) is quantised per token per 128 before the permute, the weights
 * are e4m3 codes with weights->W13_scale / W2_scale, and saved->x_perm, saved->Act hold
 * codes with saved->x_perm_scale, saved->Act_scale.
 * saved->x_perm NULL (bf16 activations, fp8 weights included): the permute only groups
 * (offsets, row_of, token_of) and the grouped fc1 reads the token rows of x (or of its
 * e4m3 codes) through saved->token_of; moe_layer_bwd then does the same for dW13.  The
 * results are bit-equal to those with the grouped copy. */
moe_status_t moe_layer_fwd(const moe_config_t* cfg, const moe_weights_t* weights, const void* x,
                           const moe_saved_t* saved, float* y, float* stats, void* ws, size_t ws_bytes,
                           void* stream);

/* ---------------------------------------------------------------- backward pieces
 * Derivatives of L = sum(dy * y) + daux * (aux + z + seq_aux); mixing weights carry the gradient to
 * the router, selection carries none ([LC] "How the router learns without an
 * expert-selection answer key"). */

/* dY_perm[row_of[t, j]] = w[t, j] * dy[t] (act dtype);  dw[t, j] = <dy[t], Y_perm[row_of[t, j]]>;
 * dY_s (NULL ok) = dy in the act dtype: the shared expert's upstream gradient; with its
 * gate (gs, Y_s and dl_s all given) dY_s = gs[t] dy[t] and
 * dl_s[t] = gs (1 - gs) <dy[t], Y_s[t]>, the gradient of the gate's logit.
 * dY_perm may be NULL when only dw is wanted (fp8 experts, whose weights are frozen). */
moe_status_t moe_unpermute_combine_bwd(const moe_config_t* cfg, const float* dy, const float* Y_perm,
                                       const int32_t* row_of, const float* w, void* dY_perm, float* dw,
                                       void* dY_s, const float* gs, const float* Y_s, float* dl_s, void* stream);

/* Expert backward, per expert e on its rows (and the shared expert on all T rows with
 * upstream gradient dY_s [T, d] act dtype, when Fs > 0):
 *   dAct = dY W2[e];  dH = [dAct * up * silu'(gate), dAct * silu(gate)];
 *   dW2[e] = dY^T Act;  dX = dH W13[e];  dW13[e] = dH^T X.
 * dX_perm (fp32) may alias dY_perm when the buffer holds A*d fp32 values (dY_perm is
 * consumed before dX_perm is written).  dH [A, 2F] and dH_s [T, 2Fs] (act dtype) are
 * outputs too.  dx_s [T, d] fp32 receives the shared expert's input gradient.
 * dW13 and dW2 may both be NULL (then dW13s and dW2s must be NULL too): only the data
 * gradients are computed, X is not read, and the weight gradients can follow from
 * moe_grouped_wgrad.  X (for dW13) is x_perm, or the token rows of x through token_of,
 * as in moe_grouped_gemm_swiglu. */
moe_status_t moe_grouped_gemm_swiglu_bwd(const moe_config_t* cfg, const void* x_perm, const int32_t* token_of,
                                         const int32_t* offsets, const void* W13, const void* W2, const void* H,
                                         const void* Act, const void* dY_perm, void* dH, void* dX_perm, void* dW13,
                                         void* dW2, const void* x, const void* W13s, const void* W2s,
                                         const void* H_s, const void* Act_s, const void* dY_s, void* dH_s,
                                         void* dx_s, void* dW13s, void* dW2s, void* ws, size_t ws_bytes,
                                         void* stream);

/* Grouped weight gradient (the expert weight gradients of [HB] §3.4's FFN, by the chain
 * rule): for each group g over its rows [offsets[g], offsets[g+1]),
 *   dW[g] = dY_g^T X_g,   fp32 accumulation, output in cfg->wgrad_dtype; overwritten
 * (accumulate = 0), or added into dW (accumulate = 1: old + the fp32 sum, one rounding
 * for bf16; a group with no rows is then left as it is).
 * dY [rows, N] and X [rows, K] in the act dtype, row-major; dW [groups, N, K].
 * The routed experts: (dH, x_perm) -> dW13 with N = 2F, K = d, and (dY_perm, Act) -> dW2
 * with N = d, K = F.  offsets NULL: one group over rows [0, rows) (the shared expert, on
 * all T tokens).  A group with no rows gets exact zeros.  offsets[groups] <= rows is the
 * caller's promise (device data is not read on the host).  One kernel launch, except:
 * ws (optional, 16-byte aligned) lets a one-group bf16 call whose dW has fewer than 128
 * tiles of 256 x 256 (a shared expert's narrow projections) split its rows into up to 8
 * chunks of at least 256 rows: fp32 partials in ws, then one kernel sums them in chunk order
 * (so the result is deterministic, and bit-equal to moe_layer_bwd's and
 * moe_grouped_gemm_swiglu_bwd's shared-expert gradients, which split the same way).  The
 * split needs chunks * N * K * 4 bytes of ws (at most 32 N K); the backward workspace of
 * moe_workspace_size covers the shared expert's two calls.  ws NULL: no split.
 * With offsets (bf16), a ws of at least moe_workspace_size's backward bytes lets the call
 * cut a group with far more rows than the others (a long-tailed routing, [HB] §3.3 Cost
 * of imbalance) into row chunks.  Its tiles would otherwise run alone on a few CUs for the
 * whole call.  The chunk is a quarter of the rows one of the kernel's tile slots holds in
 * a balanced launch (rows x tiles / slots), at least 1024.  Each chunk is an fp32 partial
 * in ws, and the partials are summed in chunk order; the other groups are computed as
 * without ws.  The split is enabled only when the chunk is below cfg->T (an expert holds
 * at most T rows) and below rows.  The plan is built on the device from offsets (no host sync).  It is the one
 * moe_layer_bwd and moe_grouped_gemm_swiglu_bwd use for the routed experts, so the call
 * gives their bits.  A ws too small for the plan: no split.
 * x_rows (bf16 activations; NULL: none): reduction row r of X is row x_rows[r] of X, which
 * then has x_src_rows rows [x_src_rows, K] (the routed dW13 straight from the token rows
 * of x, with x_rows = token_of and x_src_rows = T: bit-equal to the call on x_perm).  An
 * entry outside [0, x_src_rows) is the caller's error; the reads never leave X.
 * Errors: groups outside [1, 4096], groups != 1 without offsets, rows outside [0, 2^31),
 * N or K not a positive multiple of 64, accumulate not 0 or 1, x_rows with x_src_rows < 1
 * -> MOE_ERR_INVALID_ARG; x_rows with fp32 activations -> MOE_ERR_UNSUPPORTED; ws given
 * but smaller than a split needs -> MOE_ERR_WORKSPACE. */
moe_status_t moe_grouped_wgrad(const moe_config_t* cfg, const int32_t* offsets, int32_t groups, int64_t rows,
                               const void* dY, int32_t N, const void* X, int32_t K, const int32_t* x_rows,
                               int32_t x_src_rows, void* dW, int32_t accumulate, void* ws, size_t ws_bytes,
                               void* stream);

/* ---------------------------------------------------------------- fp8 experts
 * e4m3 block quantiser (the fp8 recipe is a reading: the pages leave low-precision expert
 * GEMMs open, [HB] §3.1 Precision asks only for an fp32 router).  src [rows, cols] is
 * bf16 (src_dtype MOE_BF16) or fp32 (MOE_F32), row-major; every block of block_rows x 128
 * gets one fp32 scale = amax / 448 computed in fp32 (1 for an all-zero block) and the
 * codes q = e4m3(v / scale): the quotient in fp32, rounded to the nearest e4m3 value
 * (ties to the even code), magnitudes above 448 saturated, sign bit = sign of v.
 * q [rows, cols] uint8; scale [rows / block_rows, cols / 128] fp32.
 * block_rows is 1 (activations: per token per 128) or 128 (weights: 128 x 128 blocks).
 * Errors: cols % 128 != 0, rows % block_rows != 0, rows < 1, other block_rows or dtypes
 * -> MOE_ERR_INVALID_ARG.  Weight quantisation for fp8 experts runs through this call
 * (one call per expert matrix, or one call over the [E*2F, d] stack). */
moe_status_t moe_quantize_fp8(int32_t src_dtype, const void* src, int64_t rows, int32_t cols, int32_t block_rows,
                              uint8_t* q, float* scale, void* stream);

/* moe_permute for e4m3 rows: the same grouping (offsets, row_of, token_of) of x_q [T, d]
 * uint8 codes into x_perm [A, d] uint8, with their scales x_scale [T, d/128] -> x_perm_scale
 * [A, d/128].  Needs cfg->w_dtype == MOE_FP8_E4M3.  x_perm and x_perm_scale both NULL: the
 * grouping only (x_q, x_scale may be NULL); one of them NULL -> MOE_ERR_INVALID_ARG. */
moe_status_t moe_permute_fp8(const moe_config_t* cfg, const uint8_t* x_q, const float* x_scale, const int32_t* idx,
                             int32_t* offsets, int32_t* row_of, int32_t* token_of, uint8_t* x_perm,
                             float* x_perm_scale, void* ws, size_t ws_bytes, void* stream);

/* Grouped SwiGLU experts with e4m3 weights and activations (cfg->w_dtype == MOE_FP8_E4M3):
 * per expert e on its rows, H = deq(x_perm) deq(W13[e])^T (fp32; the products of codes
 * accumulate on the matrix cores per 128-wide K block, then the two block scales apply);
 * Act = silu(H[:, :F]) * H[:, F:] in fp32, quantised per row per 128 columns by the rule
 * of moe_quantize_fp8 into Act [A, F] uint8 + Act_scale [A, F/128];
 * Y_perm = deq(Act) deq(W2[e])^T (fp32).  H may be NULL (not written).
 * token_of [A] (NULL: none): x_perm and x_perm_scale are then the token rows x_q [T, d] and
 * x_scale [T, d/128], and grouped row r reads token row token_of[r] (no grouped copy). */
moe_status_t moe_grouped_gemm_swiglu_fp8(const moe_config_t* cfg, const uint8_t* x_perm, const float* x_perm_scale,
                                         const int32_t* token_of, const int32_t* offsets, const uint8_t* W13,
                                         const float* W13_scale,
                                         const uint8_t* W2, const float* W2_scale, float* H, uint8_t* Act,
                                         float* Act_scale, float* Y_perm, void* ws, size_t ws_bytes, void* stream);

/* Unpermute-reduce: dx[t] = sum_j dX_perm[row_of[t, j]] (+ dx_s[t]) (+ dx_r[t])
 * (+ dl_s[t] * Wsg), fp32 accumulation in that order.  All fp32; dx_s, dx_r may be NULL;
 * dl_s and Wsg (the shared gate's input gradient) both or neither. */
moe_status_t moe_permute_bwd(const moe_config_t* cfg, const float* dX_perm, const int32_t* row_of,
                             const float* dx_s, const float* dx_r, const float* dl_s, const float* Wsg, float* dx,
                             void* stream);

/* Router backward: dlogits [T, E] from dw [T, k] through the weights of the selected
 * experts (pre_softmax: through the full softmax), plus daux times the gradients of the
 * aux loss and the sequence-wise loss through the aux probabilities (counts held
 * constant) and of the z-loss through the softmax of the logits.  counts may be NULL
 * when aux_coeff == 0 or daux == 0; seq_counts [B, E] may be NULL when seq_aux_coeff == 0
 * or daux == 0. */
moe_status_t moe_router_bwd(const moe_config_t* cfg, const float* logits, const int32_t* idx, const float* w,
                            const float* dw, const int32_t* counts, const int32_t* seq_counts, float daux,
                            float* dlogits, void* stream);

/* Gate backward: dWg = dlogits^T x [E, d]; dbg = column sums of dlogits (NULL ok);
 * dx_r = dlogits Wg [T, d] fp32 (NULL ok).  On the matrix cores like moe_gate_logits, with
 * dlogits split three ways (dWg) and both operands split (dx_r: the six part products
 * whose sum reaches fp32 precision); column sums in a fixed order.  ws as in
 * moe_gate_logits. */
moe_status_t moe_gate_logits_bwd(const moe_config_t* cfg, const void* x, const float* Wg,
                                 const float* dlogits, float* dWg, float* dbg, float* dx_r, void* ws,
                                 size_t ws_bytes, void* stream);

/* Whole backward from the saved forward tensors.
 * bf16/fp32 experts: wgrad_stream (a hipStream_t of the caller, or NULL) -- when it is
 * given and differs from `stream`, the expert weight gradients (dW2 = dY^T Act,
 * dW13 = dH^T X, routed and shared) run on it beside the data gradients: it waits on
 * `stream` for dY_perm and dH through events this call creates, and `stream` waits on it
 * before the call returns, so work queued on `stream` afterwards sees every output.  The
 * events are destroyed before the call returns; the streams are the caller's.  NULL (or
 * `stream` itself): everything runs on `stream` in order.
 * fp8 experts are frozen (no expert gradients): grads->dW13, dW2, dW13s, dW2s must be
 * NULL, and the call computes the router path only -- dw, dlogits, dWg, dbg, and
 * dx = dlogits Wg, the input gradient through the router (wgrad_stream is not used).
 * grads->accumulate = 1 adds every weight gradient into its buffer (see moe_grads_t); dx
 * is overwritten either way.  Errors: as every call, plus MOE_ERR_HIP if the events cannot
 * be created. */
moe_status_t moe_layer_bwd(const moe_config_t* cfg, const moe_weights_t* weights, const moe_saved_t* saved,
                           const void* x, const float* dy, float daux, float* dx, const moe_grads_t* grads,
                           void* ws, size_t ws_bytes, void* stream, void* wgrad_stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
