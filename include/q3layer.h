/*
 * q3layer.h -- C ABI of an MI355X (gfx950) implementation of the local
 * compute of one Qwen3 decoder layer, forward and backward.
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
 * and its backward ("each operator's backward in reverse order, locally",
 * backward table of the same page): dx and one gradient per parameter.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor arguments are DEVICE pointers to caller-owned memory; the
 *    library never allocates device memory, never synchronises, and keeps no
 *    pointer after a call returns.  Work is enqueued on `stream`, a
 *    hipStream_t passed as void* (NULL = the null stream).
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

#define Q3L_VERSION 2

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
  size_t wt;       /* bf16 only (empty for fp32): the projection weights
                      transposed to [in, out] for the backward's input-
                      gradient GEMMs: W_down^T [d_ffn, d], then [W_gate;
                      W_up]^T [d, 2*d_ffn], W_o^T [q_d, d], [W_q; W_k;
                      W_v]^T [d, q_d + 2*kv_d] (q_d = h_q*d_h, kv_d =
                      h_kv*d_h), each 256-byte aligned                    */
  size_t xnt;      /* bf16 only (empty for fp32): xn^T [d, T8] with T8 = T
                      rounded up to a multiple of 8, columns >= T zero     */
  size_t total;    /* bytes of the whole buffer                            */
} q3l_saved_layout;

/* Checks a configuration.  Q3L_OK, Q3L_EINVAL or Q3L_EUNSUPPORTED. */
q3l_status q3l_validate(const q3l_layer_cfg *cfg);

/* Fills *out with the saved-tensor layout of cfg. */
q3l_status q3l_saved_layout_of(const q3l_layer_cfg *cfg,
                               q3l_saved_layout *out);

/* Bytes of the `saved` buffer a training forward writes (0 if invalid). */
size_t q3l_saved_bytes(const q3l_layer_cfg *cfg);

/* Bytes of scratch workspace: backward == 0 for q3l_layer_forward (this
 * includes room for the intermediates when `saved` is NULL), backward == 1
 * for q3l_layer_backward.  0 if cfg is invalid. */
size_t q3l_workspace_bytes(const q3l_layer_cfg *cfg, int backward);

/* Forward of the layer (walkthrough page, Steps 1-10).
 *   x         [T, d] cfg.dtype, read only.
 *   out       where the outputs go (see q3l_outputs).
 *   saved     NULL for inference; otherwise q3l_saved_bytes(cfg) bytes that
 *             receive the intermediates q3l_layer_backward needs.  It must
 *             outlive that call, and x and the weights must not change in
 *             between.
 *   workspace q3l_workspace_bytes(cfg, 0) bytes of scratch (contents
 *             undefined afterwards); workspace_bytes is its size.
 * With bf16 and `saved`, the transposed copies (wt, xnt above) are written
 * by a second stream the library owns (one per device, created on first
 * use, default priority), forked from `stream` with an event before the
 * attention step and joined back into `stream` after it: all work of the
 * call is still ordered on `stream`, and the pattern can be captured into a
 * HIP graph. */
q3l_status q3l_layer_forward(const q3l_layer_cfg *cfg, const q3l_weights *w,
                             const void *x, const q3l_outputs *out,
                             void *saved, void *workspace,
                             size_t workspace_bytes, void *stream);

/* Backward flags.  INPUT: compute dx.  WEIGHT: compute the eleven weight
 * gradients.  ACCUMULATE: add weight gradients into the buffers instead of
 * overwriting them (gradient accumulation across micro-batches). */
enum { Q3L_BWD_INPUT = 1, Q3L_BWD_WEIGHT = 2, Q3L_BWD_ACCUMULATE = 4 };

/* Backward of the layer given dy = dLoss/dy [T, d] (cfg.dtype).
 *   saved  the buffer a forward with the same cfg, weights and x filled.
 *   dx     [T, d] cfg.dtype (written when flags & Q3L_BWD_INPUT).
 *   grads  fp32 gradient buffers (written when flags & Q3L_BWD_WEIGHT).
 *   Attention probabilities are recomputed from the saved log-sum-exp.
 *   Not available for tp_partial layers (Q3L_EUNSUPPORTED). */
q3l_status q3l_layer_backward(const q3l_layer_cfg *cfg, const q3l_weights *w,
                              const void *x, const void *dy,
                              const void *saved, void *dx,
                              const q3l_grads *grads, int flags,
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

/* y[M, N] = a[M, K] * w[N, K]^T (+ resid[M, N] if resid != NULL), the
 * bias-free linear layer of Steps 2, 6 and 9.  dtype elements; y and resid
 * may not alias a or w. */
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

/* Causal GQA attention (walkthrough page, Step 5) on one batch:
 *   q [B*L, h_q*d_h] with row stride ldq, k/v [B*L, h_kv*d_h] with row
 *   strides ldk/ldv, o [B*L, h_q*d_h] with row stride ldo (dtype);
 *   lse [B, h_q, L] fp32 (natural log).  Scale 1/sqrt(d_h).
 *   bf16: (B*L + 64) * max(ldq, ldk, ldv, ldo) * 2 and B*L*h_q*4 must stay
 *   below 2^31 (Q3L_EUNSUPPORTED otherwise; the same bound holds for
 *   q3l_attention_bwd). */
q3l_status q3l_attention_fwd(int32_t dtype, int32_t B, int32_t L,
                             int32_t h_q, int32_t h_kv, int32_t d_h,
                             const void *q, int64_t ldq, const void *k,
                             int64_t ldk, const void *v, int64_t ldv, void *o,
                             int64_t ldo, float *lse, void *stream);

/* Its backward: dq, dk, dv (dtype, same layouts/strides as q, k, v) from
 * dout (stride ldo like o), o, lse.  P is recomputed from lse.
 * workspace: q3l_attention_bwd_workspace_bytes(B, L, h_q) bytes. */
size_t q3l_attention_bwd_workspace_bytes(int32_t B, int32_t L, int32_t h_q);
q3l_status q3l_attention_bwd(int32_t dtype, int32_t B, int32_t L,
                             int32_t h_q, int32_t h_kv, int32_t d_h,
                             const void *q, int64_t ldq, const void *k,
                             int64_t ldk, const void *v, int64_t ldv,
                             const void *o, const void *dout, int64_t ldo,
                             const float *lse, void *dq, void *dk, void *dv,
                             void *workspace, size_t workspace_bytes,
                             void *stream);

#ifdef __cplusplus
}
#endif

#endif /* Q3LAYER_H */
