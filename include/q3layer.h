/*
 * q3layer.h -- C ABI of an MI355X (gfx950) implementation of the local
 * compute of one Qwen3 decoder layer, forward and backward, plus the ends of
 * the model around a stack of such layers.
 *
 * What is computed is the layer of the "FSDP2 Qwen3 Decoder Layer
 * Walkthrough" page, section "Decoder Layer 的结构" and forward Steps 1-10:
 *
 *   xn = RMSNorm(x; w_in)                          (Step 1)
 *   q, k, v = xn W_q^T, xn W_k^T, xn W_v^T         (Step 2, heads of d_h)
 *   q, k = RMSNorm_dh(q; w_qn), RMSNorm_dh(k; w_kn) (Step 3, per head)
 *   q, k = RoPE(q), RoPE(k)                         (Step 4)
 *   O = softmax(q k^T / sqrt(d_h) + causal) v       (Step 5, GQA: q head j
 *                                                    reads kv head j/(h_q/h_kv))
 *   h = x + O W_o^T                                 (Steps 6-7)
 *   y = h + W_down(silu(hn W_gate^T) * hn W_up^T),  hn = RMSNorm(h; w_post)
 *                                                   (Steps 8-10)
 *
 * and its backward (the same page's backward table: the operators' adjoints
 * run locally, last operator first): dx and one gradient per parameter.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor arguments are DEVICE pointers to caller-owned memory; the
 *    library never allocates device memory, never synchronises, holds no
 *    mutable global state (one exception: the fixed scratch array of
 *    q3l_attention_bwd_noalloc, at the end) and keeps no pointer after a
 *    call returns.  Work is
 *    enqueued on `stream`, a hipStream_t passed as void* (NULL = the null
 *    stream).  Calls on distinct buffers may run from several host threads.
 *  - Layouts are dense row-major.  Activations are [B, L, features] = [T, .]
 *    with T = B * L tokens.  Projection weights are [out, in] (nn.Linear
 *    without bias).  Head j of a projection output occupies features
 *    j*d_h .. (j+1)*d_h - 1.
 *  - dtype Q3L_BF16: activations and weights are bfloat16; GEMMs accumulate
 *    in fp32; norm statistics, softmax and log-sum-exp are fp32; weight
 *    gradients are fp32.  dtype Q3L_F32: fp32 everywhere.
 *  - Every pointer must be 16-byte aligned.  d, d_ffn must be multiples of 8;
 *    d_h is 64 or 128; h_q must be a multiple of h_kv.
 *  - Errors: each call returns a q3l_status.  Arguments are validated before
 *    anything is enqueued, so a call that fails validation writes nothing.
 *    A HIP launch error returns Q3L_EHIP.  q3l_last_error() gives a
 *    thread-local message for the last non-OK status.  Nothing aborts.
 */
#ifndef Q3LAYER_H
#define Q3LAYER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q3L_VERSION 3

typedef enum { Q3L_F32 = 0, Q3L_BF16 = 1 } q3l_dtype;

typedef enum {
  Q3L_OK = 0,
  Q3L_EINVAL = 1,       /* bad shape, null pointer, too-small workspace  */
  Q3L_EUNSUPPORTED = 2, /* valid layer, but not one this build supports  */
  Q3L_EALIGN = 3,       /* a pointer is not 16-byte aligned              */
  Q3L_EHIP = 4          /* a HIP call failed                              */
} q3l_status;

/* Layer hyper-parameters (the walkthrough page's configuration table plus
 * the numerics the page leaves symbolic). */
typedef struct {
  int32_t d;        /* hidden size                                       */
  int32_t h_q;      /* query heads                                       */
  int32_t h_kv;     /* key/value heads (GQA; h_q % h_kv == 0)            */
  int32_t d_h;      /* head dim: 64 or 128                               */
  int32_t d_ffn;    /* SwiGLU intermediate size                          */
  int32_t B;        /* sequences                                         */
  int32_t L;        /* tokens per sequence (positions 0..L-1)            */
  float eps;        /* RMSNorm epsilon, inside the square root           */
  float rope_theta; /* RoPE base                                         */
  int32_t qk_norm;  /* 1: Qwen3 per-head q_norm/k_norm (Step 3); 0: none  */
  int32_t tp_partial; /* 1: one tensor-parallel rank's share -- o_proj and
                         down_proj write fp32 partial sums (no reduction);
                         h = x + attn_partial feeds the MLP.  Forward only. */
  int32_t dtype;    /* q3l_dtype                                         */
} q3l_layer_cfg;

/* The eleven parameters, in the walkthrough page's table order.  Pointers
 * to cfg.dtype elements: in_norm[d], q[h_q*d_h, d], k[h_kv*d_h, d],
 * v[h_kv*d_h, d], q_norm[d_h], k_norm[d_h], o[d, h_q*d_h], post_norm[d],
 * gate[d_ffn, d], up[d_ffn, d], down[d, d_ffn]. */
typedef struct {
  const void *in_norm, *q, *k, *v, *q_norm, *k_norm, *o, *post_norm, *gate,
      *up, *down;
} q3l_weights;

/* fp32 gradient buffers with the same shapes as q3l_weights. */
typedef struct {
  float *in_norm, *q, *k, *v, *q_norm, *k_norm, *o, *post_norm, *gate, *up,
      *down;
} q3l_grads;

/* Forward outputs.  y [T, d] (cfg.dtype) when tp_partial == 0; otherwise
 * attn_partial [T, d] and mlp_partial [T, d], fp32. */
typedef struct {
  void *y;
  float *attn_partial;
  float *mlp_partial;
} q3l_outputs;

/* Byte offsets of the tensors the forward saves for the backward, inside the
 * caller's `saved` buffer (each 256-byte aligned).  Exposed so callers and
 * tests can inspect intermediates. */
typedef struct {
  size_t rstd1;    /* [T] fp32, 1/rms of x                                 */
  size_t xn;       /* [T, d] dtype, RMSNorm(x; w_in)                       */
  size_t qkv;      /* [T, h_q*d_h + 2*h_kv*d_h] dtype: q, k before the
                      q/k norm, and v                                      */
  size_t qk_rope;  /* [T, h_q*d_h + h_kv*d_h] dtype: q, k after norm+RoPE   */
  size_t rstd_q;   /* [T, h_q] fp32                                        */
  size_t rstd_k;   /* [T, h_kv] fp32                                       */
  size_t rope_cos; /* [L, d_h/2] fp32                                      */
  size_t rope_sin; /* [L, d_h/2] fp32                                      */
  size_t attn_o;   /* [T, h_q*d_h] dtype, attention output                 */
  size_t lse;      /* [B, h_q, L] fp32, natural-log sum of exp of scores   */
  size_t h;        /* [T, d] dtype, x + attention branch                   */
  size_t rstd2;    /* [T] fp32                                             */
  size_t hn;       /* [T, d] dtype, RMSNorm(h; w_post)                     */
  size_t gu;       /* [T, 2*d_ffn] dtype: gate in columns [0, d_ffn), up in
                      [d_ffn, 2*d_ffn)                                     */
  size_t f;        /* [T, d_ffn] dtype, silu(gate) * up                    */
  size_t wt;       /* empty (wt == xnt): the backward's input-gradient
                      GEMMs read the projection weights as they are       */
  size_t xnt;      /* bf16 with tp_partial == 0 only (else empty): xn^T
                      [d, T8] with T8 = T rounded up to a multiple of 8,
                      columns >= T zero (the QKV weight gradient's operand) */
  size_t total;    /* bytes of the whole buffer                            */
} q3l_saved_layout;

/* Execution options of q3l_layer_forward / q3l_layer_backward.  Pass NULL
 * for the defaults: every kernel on `stream` and no phase marks.  Every
 * object named here is created and owned by the caller. */
typedef struct {
  /* Optional second stream for work that depends only on the call's inputs:
   * the bf16 training forward's transposed copy (saved xnt), which
   * then runs beside the attention step.  NULL: it runs on `stream`.  When
   * set, fork_event and join_event must be hipEvent_t the caller created
   * (timing may be disabled).  The call records fork_event on `stream`,
   * makes side_stream wait for it, enqueues the copy on side_stream,
   * records join_event there and, at the end of the forward (after the last
   * phase mark, and on every error path once the join event is recorded),
   * makes `stream` wait for it: all work of the call stays ordered on
   * `stream` (and can be captured into a HIP graph).
   * Calls that share these objects must not be made concurrently. */
  void *side_stream;
  void *fork_event;
  void *join_event;
  /* Optional phase marks: NULL, or q3l_phase_count(pass) + 1 hipEvent_t
   * created by the caller with timing enabled.  marks[0] is recorded on
   * `stream` before the first kernel of the call and marks[i + 1] after
   * phase i (phases a call skips are empty), so the elapsed time between
   * marks[i] and marks[i + 1] is phase i's time on the stream. */
  void *const *marks;
  int32_t n_marks;
} q3l_exec;

/* Number of phases of a forward (backward == 0) or backward (1) call, and
 * the name of phase i ("F5 attention", ...; NULL out of range). */
int q3l_phase_count(int backward);
const char *q3l_phase_name(int backward, int i);

/* Checks a configuration.  Q3L_OK, Q3L_EINVAL or Q3L_EUNSUPPORTED. */
q3l_status q3l_validate(const q3l_layer_cfg *cfg);

/* Fills *out with the saved-tensor layout of cfg. */
q3l_status q3l_saved_layout_of(const q3l_layer_cfg *cfg,
                               q3l_saved_layout *out);

/* Bytes of the `saved` buffer a training forward writes (0 if invalid). */
size_t q3l_saved_bytes(const q3l_layer_cfg *cfg);

/* Bytes of scratch workspace: backward == 0 for q3l_layer_forward (this
 * includes room for the intermediates when `saved` is NULL), backward == 1
 * for q3l_layer_backward.  0 if cfg is invalid.  The bf16 backward's includes
 * the attention backward's dS (see q3l_attention_bwd) while that stays
 * within 8 GiB (about B h_q L^2 bytes; 1.08 GB at B = 2, L = 4096, 32 q
 * heads); beyond, the attention backward recomputes S and dP for dQ. */
size_t q3l_workspace_bytes(const q3l_layer_cfg *cfg, int backward);

/* Forward of the layer (walkthrough page, Steps 1-10).
 *   x         [T, d] cfg.dtype, read only.
 *   out       where the outputs go (see q3l_outputs).
 *   saved     NULL for inference; otherwise q3l_saved_bytes(cfg) bytes that
 *             receive the intermediates q3l_layer_backward needs.  It must
 *             outlive that call, and x and the weights must not change in
 *             between.
 *   workspace q3l_workspace_bytes(cfg, 0) bytes of scratch (contents
 *             undefined afterwards); workspace_bytes is its size.  Only
 *             needed (and only checked) when saved is NULL.
 *   exec      NULL or execution options (see q3l_exec). */
q3l_status q3l_layer_forward(const q3l_layer_cfg *cfg, const q3l_weights *w,
                             const void *x, const q3l_outputs *out,
                             void *saved, void *workspace,
                             size_t workspace_bytes, void *stream,
                             const q3l_exec *exec);

/* Backward flags.  INPUT: compute dx.  WEIGHT: compute the eleven weight
 * gradients.  ACCUMULATE: add weight gradients into the buffers instead of
 * overwriting them (gradient accumulation across micro-batches).
 * DEFERRED_WEIGHT (with WEIGHT, without INPUT): the input-gradient half of
 * the backward was already run by an INPUT-only call on the same workspace
 * (same cfg, weights, x, dy and saved), which leaves the activation
 * gradients and the norm-weight partial sums there; only the weight-
 * gradient GEMMs (with their operand transposes) and the norm-weight
 * reductions run.  This is the split of the backward into an input-gradient
 * part B and a weight-gradient part W of the parallelism page's pipeline
 * section (zero-bubble schedules): INPUT then WEIGHT|DEFERRED_WEIGHT gives
 * bitwise the results of one INPUT|WEIGHT call. */
enum {
  Q3L_BWD_INPUT = 1,
  Q3L_BWD_WEIGHT = 2,
  Q3L_BWD_ACCUMULATE = 4,
  Q3L_BWD_DEFERRED_WEIGHT = 8
};

/* Backward of the layer given dy = dLoss/dy [T, d] (cfg.dtype).
 *   saved     the buffer a forward with the same cfg, weights and x filled.
 *   dx        [T, d] cfg.dtype (written when flags & Q3L_BWD_INPUT).
 *   grads     fp32 gradient buffers (written when flags & Q3L_BWD_WEIGHT).
 *   workspace q3l_workspace_bytes(cfg, 1) bytes; between an INPUT-only call
 *             and its DEFERRED_WEIGHT call it must not be reused.
 *   Attention probabilities are recomputed from the saved log-sum-exp.
 *   Not available for tp_partial layers (Q3L_EUNSUPPORTED). */
q3l_status q3l_layer_backward(const q3l_layer_cfg *cfg, const q3l_weights *w,
                              const void *x, const void *dy,
                              const void *saved, void *dx,
                              const q3l_grads *grads, int flags,
                              void *workspace, size_t workspace_bytes,
                              void *stream, const q3l_exec *exec);

/* ------------------------------------------------------------------------
 * The model around a stack of layers (walkthrough page, "简化的 Qwen3 结构":
 * embed_tokens [vocab, d], N_L decoder layers, a final RMSNorm, and an
 * output projection tied to the embedding; hidden states flow from one
 * layer into the next on the same device, the text after Steps 10-11):
 *   x_0 = E[ids];  x_{i+1} = layer_i(x_i);  hf = RMSNorm(x_N; w_final);
 *   logits = hf E^T.
 * The loss is not part of the path: the backward starts from dlogits.
 * ------------------------------------------------------------------------ */
typedef struct {
  q3l_layer_cfg layer; /* shapes and numerics of every layer (tp_partial 0) */
  int32_t n_layers;    /* N_L >= 0                                         */
  int32_t vocab;       /* V: rows of the embedding table, a multiple of 8  */
  int32_t recompute;   /* 1: the forward keeps only each layer's input and
                          the backward recomputes each layer's forward before
                          its backward (the memory-model page's full
                          recompute, section 3.3: one more forward, far less
                          saved memory); 0: every layer's saved block is
                          kept                                            */
} q3l_model_cfg;

typedef struct {
  const void *embed;         /* [V, d] cfg dtype, also the output projection */
  const void *final_norm;    /* [d] cfg dtype                               */
  const q3l_weights *layers; /* host array of n_layers (device pointers)    */
} q3l_model_weights;

typedef struct {
  float *embed;              /* [V, d] fp32: output projection + embedding  */
  float *final_norm;         /* [d] fp32                                    */
  const q3l_grads *layers;   /* host array of n_layers                      */
} q3l_model_grads;

/* Checks a model configuration (the layer's rules, V a positive multiple of
 * 8, n_layers >= 0, B*L <= 262144 tokens, and in bf16 the logits and the
 * table within the GEMM's 2 GiB offset range). */
q3l_status q3l_model_validate(const q3l_model_cfg *cfg);
/* Bytes of the `saved` buffer of a training forward (layer inputs, the
 * final norm's output and statistics, and -- without recompute -- every
 * layer's saved block); 0 if invalid. */
size_t q3l_model_saved_bytes(const q3l_model_cfg *cfg);
/* Bytes of scratch of q3l_model_forward (backward == 0) or
 * q3l_model_backward (1); 0 if invalid. */
size_t q3l_model_workspace_bytes(const q3l_model_cfg *cfg, int backward);

/* Forward: ids [B*L] int32 device array (ids outside [0, V) embed as zero
 * rows); logits [B*L, V] cfg dtype.  saved: NULL for inference, else
 * q3l_model_saved_bytes(cfg) bytes kept for the backward.  exec: NULL, or
 * options whose side_stream (and its events) each layer's forward uses;
 * exec->marks must be NULL here. */
q3l_status q3l_model_forward(const q3l_model_cfg *cfg,
                             const q3l_model_weights *w, const int32_t *ids,
                             void *logits, void *saved, void *workspace,
                             size_t workspace_bytes, void *stream,
                             const q3l_exec *exec);

/* Backward from dlogits [B*L, V] (cfg dtype): every gradient of the stack,
 * fp32, overwritten (flags 0) or added into (Q3L_BWD_ACCUMULATE).  The
 * embedding table's gradient is the output projection's weight gradient
 * plus, for every token, its row of dx_0 scattered into the token's row (in
 * a fixed order: bitwise reproducible). */
q3l_status q3l_model_backward(const q3l_model_cfg *cfg,
                              const q3l_model_weights *w, const int32_t *ids,
                              const void *dlogits, const void *saved,
                              const q3l_model_grads *grads, int flags,
                              void *workspace, size_t workspace_bytes,
                              void *stream);

/* Thread-local text describing the last non-OK status ("" if none). */
const char *q3l_last_error(void);

/* Q3L_VERSION of the built library. */
int q3l_version(void);

/* ------------------------------------------------------------------------
 * Phase-level entry points: one step of the layer each, with the same
 * conventions, for per-step tests and timing.  Row strides are in elements.
 * ------------------------------------------------------------------------ */

/* RMSNorm over rows (walkthrough page, Step 1 formula):
 *   y[r, :] = x[r, :] / sqrt(mean(x[r, :]^2) + eps) * w,  rstd[r] = that
 *   reciprocal (fp32).  x, y: [rows, n] dtype; w: [n] dtype; n a multiple
 *   of 8 and at most 8192 (Q3L_EUNSUPPORTED beyond). */
q3l_status q3l_rmsnorm_fwd(int32_t dtype, int64_t rows, int32_t n,
                           const void *x, const void *w, float eps, void *y,
                           float *rstd, void *stream);

/* Adjoint of q3l_rmsnorm_fwd (walkthrough page, backward of Steps 1 and 8),
 * given the forward's x and rstd:
 *   dx[r, :] = rstd (g - xhat mean(g xhat)) + resid[r, :],
 *   with xhat = x rstd and g = dy w;   dw (+)= sum_r dy[r, :] xhat[r, :].
 * dy, x, resid (optional, may be NULL), dx: [rows, n] dtype; w [n] dtype;
 * dw [n] fp32 (optional: NULL computes dx only), overwritten, or added into
 * when accumulate != 0; the sum over rows has a fixed order.  workspace:
 * q3l_rmsnorm_bwd_workspace_bytes(n) bytes of scratch (partial sums of dw).
 * n as for q3l_rmsnorm_fwd. */
size_t q3l_rmsnorm_bwd_workspace_bytes(int32_t n);
q3l_status q3l_rmsnorm_bwd(int32_t dtype, int64_t rows, int32_t n,
                           const void *dy, const void *x, const float *rstd,
                           const void *w, const void *resid, void *dx,
                           float *dw, int accumulate, void *workspace,
                           size_t workspace_bytes, void *stream);

/* RoPE angle table (walkthrough page, Step 4): for position t < L and pair
 * i < d_h/2, angle t * theta^(-2i/d_h) (computed in double), cos_t[t, i] and
 * sin_t[t, i] fp32 [L, d_h/2].  The pairing is rotate-half: element i of a
 * head vector pairs with element i + d_h/2. */
q3l_status q3l_rope_table(int32_t L, int32_t d_h, float theta, float *cos_t,
                          float *sin_t, void *stream);

/* Steps 3-4 of the walkthrough page in one pass: for every token t (position
 * t % L) and every head of a [B*L, ld_in] buffer whose columns hold h_q
 * query heads then h_kv key heads of d_h each, the per-head RMSNorm over d_h
 * with weight wq (query heads) or wk (key heads) -- skipped when
 * qk_norm == 0 -- then the rotation by the angles of q3l_rope_table:
 *   out[i] = n[i] cos - n[i + d_h/2] sin,  out[i + d_h/2] = n[i + d_h/2] cos
 *   + n[i] sin   (i < d_h/2).
 * out has the same column arrangement with row stride ld_out; rstd_q
 * [B*L, h_q] and rstd_k [B*L, h_kv] fp32 receive the norms' reciprocal
 * rms (unused when qk_norm == 0). */
q3l_status q3l_qknorm_rope_fwd(int32_t dtype, int32_t B, int32_t L,
                               int32_t h_q, int32_t h_kv, int32_t d_h,
                               int32_t qk_norm, float eps, const void *in,
                               int64_t ld_in, const void *wq, const void *wk,
                               const float *cos_t, const float *sin_t,
                               void *out, int64_t ld_out, float *rstd_q,
                               float *rstd_k, void *stream);

/* Adjoint of q3l_qknorm_rope_fwd: g (gradient w.r.t. its output, stride
 * ld_g) is rotated back (the rotation by the opposite angle), then taken
 * through the per-head RMSNorm given the forward's input `pre` (stride
 * ld_pre) and rstd_q / rstd_k; out (stride ld_out) receives the gradient
 * w.r.t. the forward's input.  dwq, dwk [d_h] fp32 (overwritten, or added
 * into when accumulate != 0; NULL skips) receive the norm weights'
 * gradients summed over tokens and heads in a fixed order.  workspace:
 * q3l_qknorm_rope_bwd_workspace_bytes(d_h) bytes of scratch. */
size_t q3l_qknorm_rope_bwd_workspace_bytes(int32_t d_h);
q3l_status q3l_qknorm_rope_bwd(int32_t dtype, int32_t B, int32_t L,
                               int32_t h_q, int32_t h_kv, int32_t d_h,
                               int32_t qk_norm, const void *g, int64_t ld_g,
                               const void *pre, int64_t ld_pre,
                               const void *wq, const void *wk,
                               const float *rstd_q, const float *rstd_k,
                               const float *cos_t, const float *sin_t,
                               void *out, int64_t ld_out, float *dwq,
                               float *dwk, int accumulate, void *workspace,
                               size_t workspace_bytes, void *stream);

/* y[M, N] = a[M, K] * w[N, K]^T (+ resid[M, N] if resid != NULL), the
 * bias-free linear layer of Steps 2, 6 and 9.  dtype elements; y and resid
 * may not alias a or w.  bf16: (M + 8) * max(N, K) * 2 and (N + 8) * K * 2
 * bytes must stay below 2^31 (Q3L_EUNSUPPORTED beyond; the same holds for
 * the dgrad, wgrad and SwiGLU calls below). */
q3l_status q3l_linear_fwd(int32_t dtype, int64_t M, int32_t N, int32_t K,
                          const void *a, const void *w, const void *resid,
                          void *y, void *stream);

/* Input gradient of a linear layer: da[M, K] = dy[M, N] * w[N, K]. */
q3l_status q3l_linear_dgrad(int32_t dtype, int64_t M, int32_t N, int32_t K,
                            const void *dy, const void *w, void *da,
                            void *stream);

/* Weight gradient of a linear layer, fp32:
 *   dw[N, K] (+)= dy[M, N]^T * a[M, K]   (sum over the M tokens);
 *   accumulate != 0 adds into dw. */
q3l_status q3l_linear_wgrad(int32_t dtype, int64_t M, int32_t N, int32_t K,
                            const void *dy, const void *a, float *dw,
                            int accumulate, void *stream);

/* First half of Step 9 (walkthrough page, SwiGLU MLP) as one fused GEMM:
 *   g = hn gate^T, u = hn up^T, f = silu(g) * u
 * hn [M, K], gate/up [N, K], f [M, N] (dtype).  gu (optional, may be NULL)
 * receives g in columns [0, N) and u in [N, 2N) of a [M, 2N] buffer.  This is
 * the kernel the layer forward launches for that step. */
q3l_status q3l_swiglu_fwd(int32_t dtype, int64_t M, int32_t N, int32_t K,
                          const void *hn, const void *gate, const void *up,
                          void *f, void *gu, void *stream);

/* Adjoint of f = silu(g) * u (walkthrough page, Step 9), with s = sigmoid(g):
 *   dg = df u s (1 + g (1 - s)),  du = df g s.
 * df [M, N]; gu [M, 2N] holds g in columns [0, N) and u in [N, 2N); dgu
 * [M, 2N] receives dg then du (dtype; N a multiple of 8).  dgu may not
 * alias gu; it may alias df only when df is dgu's dg half (row stride 2N,
 * which this call does not take: pass distinct buffers). */
q3l_status q3l_swiglu_bwd(int32_t dtype, int64_t M, int32_t N, const void *df,
                          const void *gu, void *dgu, void *stream);

/* Causal GQA attention (walkthrough page, Step 5) on one batch:
 *   q [B*L, h_q*d_h] with row stride ldq, k/v [B*L, h_kv*d_h] with row
 *   strides ldk/ldv, o [B*L, h_q*d_h] with row stride ldo (dtype);
 *   lse [B, h_q, L] fp32 (natural log).  Scale 1/sqrt(d_h).
 *   bf16: (B*L + 64) * max(ldq, ldk, ldv, ldo) * 2 and B*L*h_q*4 must stay
 *   below 2^31 (Q3L_EUNSUPPORTED otherwise; the same bound holds for
 *   q3l_attention_bwd with its strides). */
q3l_status q3l_attention_fwd(int32_t dtype, int32_t B, int32_t L,
                             int32_t h_q, int32_t h_kv, int32_t d_h,
                             const void *q, int64_t ldq, const void *k,
                             int64_t ldk, const void *v, int64_t ldv, void *o,
                             int64_t ldo, float *lse, void *stream);

/* Attention over one block of keys, as the parallelism page's ring-attention
 * section (4.2) builds it: for every sequence b, q head j and query t, over
 * the keys s in [k0, k1) with s <= t (positions within the sequence; the
 * causal rule of Step 5), with S = q k / sqrt(d_h):
 *   m = max S (the block's largest score), l = sum exp(S - m),
 *   acc = sum exp(S - m) v_s   (unnormalised, fp32),
 * and (-inf, 0, 0) for a query that sees no key of the block.  q, k, v as
 * for q3l_attention_fwd; m, l [B, h_q, L] fp32; acc [B*L, h_q*d_h] fp32
 * (dense).  0 <= k0 < k1 <= L.  States of disjoint key blocks combine with
 * q3l_attention_merge, in any order, to the state of their union; the
 * merged state of a partition of [0, L) gives the attention output through
 * q3l_attention_finish. */
q3l_status q3l_attention_fwd_block(int32_t dtype, int32_t B, int32_t L,
                                   int32_t h_q, int32_t h_kv, int32_t d_h,
                                   const void *q, int64_t ldq, const void *k,
                                   int64_t ldk, const void *v, int64_t ldv,
                                   int32_t k0, int32_t k1, float *m, float *l,
                                   float *acc, void *stream);

/* The merge rule of the same section, in place: with m_new = max(m, m2),
 * l = l e^(m - m_new) + l2 e^(m2 - m_new), acc likewise, m = m_new (a
 * (-inf, 0, 0) state drops out).  Layouts as q3l_attention_fwd_block. */
q3l_status q3l_attention_merge(int32_t B, int32_t L, int32_t h_q, int32_t d_h,
                               float *m, float *l, float *acc, const float *m2,
                               const float *l2, const float *acc2,
                               void *stream);

/* The output of a (merged) state: o = acc / l (dtype, row stride ldo) and
 * lse = m + log l (natural log, [B, h_q, L] fp32; -inf and o = 0 where l is
 * 0). */
q3l_status q3l_attention_finish(int32_t dtype, int32_t B, int32_t L,
                                int32_t h_q, int32_t d_h, const float *m,
                                const float *l, const float *acc, void *o,
                                int64_t ldo, float *lse, void *stream);

/* Its backward: dq, dk, dv (dtype) are written with the row strides of q, k,
 * v (ldq, ldk, ldv) -- a caller that passes strided views must give dq, dk,
 * dv buffers of the same strides -- from o (stride ldo), dout (stride
 * lddo) and lse.  P is recomputed from lse.  workspace: at least
 * q3l_attention_bwd_workspace_bytes(B, L, h_q) bytes of scratch (the row
 * sums of dout * o).  bf16 with at least
 * q3l_attention_bwd_stored_ds_workspace_bytes(B, L, h_q) bytes (the row
 * sums plus dS for the causal triangle in 32 x 32 bf16 blocks, about
 * B h_q L^2 bytes): the dK/dV kernel also stores dS = P (dP - D) and dQ =
 * dS K / sqrt(d_h) is formed from it, instead of a second kernel that
 * recomputes S and dP (the walkthrough page's backward section: each
 * operator's local gradient; the same values, computed once).  The results
 * are bitwise the same either way. */
size_t q3l_attention_bwd_workspace_bytes(int32_t B, int32_t L, int32_t h_q);
size_t q3l_attention_bwd_stored_ds_workspace_bytes(int32_t B, int32_t L,
                                                   int32_t h_q);
q3l_status q3l_attention_bwd(int32_t dtype, int32_t B, int32_t L,
                             int32_t h_q, int32_t h_kv, int32_t d_h,
                             const void *q, int64_t ldq, const void *k,
                             int64_t ldk, const void *v, int64_t ldv,
                             const void *o, int64_t ldo, const void *dout,
                             int64_t lddo, const float *lse, void *dq,
                             void *dk, void *dv, void *workspace,
                             size_t workspace_bytes, void *stream);

/* q3l_attention_bwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without a workspace.  The row-sum scratch
 * comes from a fixed device array inside the library, one per GPU, held
 * until the process ends: B*h_q*L may not exceed
 * q3l_attention_bwd_noalloc_max_rows() (4,194,304; Q3L_EINVAL beyond, before
 * anything is enqueued).  The call allocates nothing.  All calls on one GPU
 * share that array, so calls that overlap on one GPU (concurrent streams or
 * host threads) race and must be serialised by the caller; results are
 * bitwise those of q3l_attention_bwd. */
size_t q3l_attention_bwd_noalloc_max_rows(void);
q3l_status q3l_attention_bwd_noalloc(int32_t dtype, int32_t B, int32_t L,
                                     int32_t h_q, int32_t h_kv, int32_t d_h,
                                     const void *q, int64_t ldq, const void *k,
                                     int64_t ldk, const void *v, int64_t ldv,
                                     const void *o, int64_t ldo,
                                     const void *dout, int64_t lddo,
                                     const float *lse, void *dq, void *dk,
                                     void *dv, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* Q3LAYER_H */
