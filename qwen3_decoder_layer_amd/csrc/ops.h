// Internal launch interface between the host orchestration (api.cpp) and the
// kernels.  Every launcher enqueues on `s` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q3l {

// A GEMM operand viewed as a [rows x K] matrix that is staged into LDS with K
// contiguous.  Two storage forms:
//  - k_contig = 1: element (r, k) at p[s][(r - start[s]) * ld[s] + k], the
//    segment s chosen by r (weights stored [out, in], activations [T, f]).
//    paired = 1 interleaves two segments in 32-row blocks: logical row r
//    reads segment (r / 32) % 2, row (r / 64) * 32 + r % 32 (the gate/up pair).
//  - k_contig = 0: element (r, k) at p[s][(k - start[s]) * ld[s] + r], the
//    segment s chosen by k (a weight read as [in, out], or activations read
//    transposed for a weight gradient).
struct Operand {
  const void* p[3];
  int64_t ld[3];
  int32_t start[3];
  int32_t nseg;
  int32_t rows;      // valid rows (for paired: rows of ONE segment)
  int32_t k_contig;
  int32_t paired;
};

enum EpiKind : int32_t {
  EPI_STORE = 0,     // C = acc (+ R)                      dtype C, R
  EPI_PARTIAL = 1,   // P = acc fp32; H = R + acc (opt.)    fp32 P, dtype H
  EPI_SILU_MUL = 2,  // paired gate/up: G|U (opt.), F = silu(g) * u
  EPI_SILU_BWD = 3,  // df tile + saved g, u -> dg, du
  EPI_WGRAD = 4      // fp32 C (+)= acc, C split by M segments
};

struct Epilogue {
  int32_t kind;
  void* c;          // STORE: C; PARTIAL: H (may be null); SILU_MUL: F;
                    // SILU_BWD: dG|dU base
  int64_t ldc;
  const void* r;    // STORE / PARTIAL: residual (may be null);
                    // SILU_BWD: saved G|U base
  int64_t ldr;
  float* p32;       // PARTIAL: fp32 partial
  int64_t ldp;
  void* gu;         // SILU_MUL: saved G|U base (may be null)
  int64_t ldgu;
  int32_t ffn;      // SILU_*: d_ffn (U starts at column ffn of G|U)
  // WGRAD
  float* cs[3];
  int32_t cstart[3];
  int32_t cnseg;
  int32_t accumulate;
};

struct GemmArgs {
  Operand a, b;       // C[M, N] = sum_k A(m, k) B(n, k)
  int32_t M, N, K;    // N is the logical width (paired: 2 * round_up(ffn, 32))
  Epilogue epi;
};

// bf16 MFMA GEMM (K must be a multiple of 8; every k_contig = 0 operand's
// rows a multiple of 8).  Operand forms: both K-contiguous, A K-contiguous
// with B row-contiguous, or both row-contiguous; A row-contiguous with B
// K-contiguous returns hipErrorInvalidValue.
hipError_t gemm_bf16(const GemmArgs& g, hipStream_t s);
// Plain fp32 GEMM with the same argument structure (correctness path).
hipError_t gemm_f32(const GemmArgs& g, hipStream_t s);

// bf16 dst[c][r] = src[r][c] (r < rows, c < cols); dst columns r in
// [rows, rows_pad) are zero.  rows_pad and cols multiples of 8.
hipError_t transpose_bf16(int rows, int rows_pad, int cols, const void* src,
                          int64_t ld_src, void* dst, int64_t ld_dst, hipStream_t s);
// Up to kTransposeBatchMax transposes in one launch (jobs with no work are
// skipped).
constexpr int kTransposeBatchMax = 8;
struct TransposeJob {
  const void* src; int64_t ld_src;
  void* dst; int64_t ld_dst;
  int rows, rows_pad, cols;
};
hipError_t transpose_bf16_batch(const TransposeJob* jobs, int n, hipStream_t s);

// SwiGLU adjoint, bf16: from df [T, ffn] and the saved g|u [T, 2 ffn] write
// dgu = [dg | du] ([T, 2 ffn]) and, if dguT is not null, its transpose dguT
// ([2 ffn, Tp], columns t >= T zero).  df may alias the dg half of dgu (same
// ld).  ffn and Tp multiples of 8.
hipError_t swiglu_bwd_bf16(int T, int Tp, int ffn, const void* df, int64_t ld_df,
                           const void* gu, int64_t ld_gu, void* dgu, int64_t ld_dgu,
                           void* dguT, int64_t ld_t, hipStream_t s);
// Only the transposed copy of the above, from a dgu an earlier
// swiglu_bwd_bf16 wrote: bitwise the dguT the fused form writes.
hipError_t swiglu_transposes_bf16(int T, int Tp, int ffn, const void* dgu, int64_t ld_dgu,
                                  void* dguT, int64_t ld_t, hipStream_t s);
// fp32 SwiGLU adjoint, dgu = [dg | du] from df and g | u.
hipError_t swiglu_bwd_f32(int64_t M, int ffn, const float* df, int64_t ld_df, const float* gu,
                          int64_t ld_gu, float* dgu, int64_t ld_dgu, hipStream_t s);

// ---- norms / RoPE / elementwise (dtype: 0 fp32, 1 bf16) -------------------
hipError_t rmsnorm_fwd(int dtype, int64_t rows, int n, const void* x,
                       const void* w, float eps, void* y, float* rstd,
                       hipStream_t s);
// dx = resid + rmsnorm_backward(dy);  dw partial sums per block into
// wpart[nblocks_out][n] (fp32).  Returns the number of partial rows written
// through *nparts.  resid (optional) and dx are dtype.
hipError_t rmsnorm_bwd(int dtype, int64_t rows, int n, const void* dy,
                       const void* x, const float* rstd, const void* w,
                       const void* resid, void* dx, float* wpart, int* nparts,
                       hipStream_t s);
int rmsnorm_bwd_max_parts();
// The partial-row count rmsnorm_bwd reports for these sizes.
int rmsnorm_bwd_parts(int dtype, int64_t rows, int n);
// out[n] (+)= sum_p part[p][n]
hipError_t reduce_rows(const float* part, int nparts, int n, float* out,
                       int accumulate, hipStream_t s);
// Two reductions of the same shape in one launch: out (+)= rows of part,
// out2 (+)= rows of part2.
hipError_t reduce_rows2(const float* part, const float* part2, int nparts, int n,
                        float* out, float* out2, int accumulate, hipStream_t s);
hipError_t rope_table(int L, int d_h, float theta, float* cos_t, float* sin_t,
                      hipStream_t s);
// q/k norm + RoPE over the q and k heads of a [T, ld_in] buffer.
hipError_t qknorm_rope_fwd(int dtype, int B, int L, int h_q, int h_kv,
                           int d_h, int qk_norm, float eps, const void* in,
                           int64_t ld_in, const void* wq, const void* wk,
                           const float* cos_t, const float* sin_t, void* out,
                           int64_t ld_out, float* rstd_q, float* rstd_k,
                           hipStream_t s);
hipError_t qknorm_rope_bwd(int dtype, int B, int L, int h_q, int h_kv,
                           int d_h, int qk_norm, const void* g_in,
                           int64_t ld_g, const void* pre, int64_t ld_pre,
                           const void* wq, const void* wk, const float* rstd_q,
                           const float* rstd_k, const float* cos_t,
                           const float* sin_t, void* out, int64_t ld_out,
                           float* wq_part, float* wk_part, int* nparts,
                           hipStream_t s);
int qknorm_bwd_max_parts();
// The partial-row count qknorm_rope_bwd reports (heads = h_q + h_kv).
int qknorm_bwd_parts(int64_t tokens, int heads, int d_h);

// ---- token embedding ------------------------------------------------------
// x[t] = E[ids[t]] (zero rows for ids outside [0, V)); d a multiple of 8.
hipError_t embed_gather(int dtype, int64_t T, int d, int V, const int32_t* ids, const void* E,
                        void* x, hipStream_t s);
// dE[v] += sum over t with ids[t] = v of dx[t] (fp32, fixed order); next and
// first are [T] int32 scratch.  d <= 8192.
hipError_t embed_scatter_add(int dtype, int T, int d, int V, const int32_t* ids,
                             const void* dx, int32_t* next, int32_t* first, float* dE,
                             hipStream_t s);

// ---- attention ------------------------------------------------------------
struct AttnArgs {
  int B, L, h_q, h_kv, d_h;
  const void* q; int64_t ldq;
  const void* k; int64_t ldk;
  const void* v; int64_t ldv;
  void* o; int64_t ldo;
  float* lse;
  // backward only
  const void* dout; int64_t lddo;
  void* dq; void* dk; void* dv;   // strides ldq / ldk / ldv
  float* delta;                   // [B, h_q, L] scratch
  // bf16: attn_ds_bytes(B, L, h_q) bytes of scratch for the stored-dS form
  // (dQ formed from dS written by the dK/dV kernel), or null to recompute
  // S and dP for dQ instead.  Results are the same either way.
  void* ds;
  // block state only: keys [k_lo, k_hi); m, l [B, h_q, L]; acc [B*L, ld_acc]
  int k_lo, k_hi;
  float* m_out; float* l_out; float* acc; int64_t ld_acc;
};
hipError_t attn_fwd(int dtype, const AttnArgs& a, hipStream_t s);
hipError_t attn_bwd(int dtype, const AttnArgs& a, hipStream_t s);
// 32x32 dS blocks of the causal triangle per (sequence, q head), and the
// bytes of the stored-dS scratch.
inline int64_t attn_ds_blocks(int L) {
  const int64_t n = (L + 31) / 32;
  return n * (n + 1) / 2;
}
inline size_t attn_ds_bytes(int B, int L, int h_q) {
  return (size_t)B * h_q * (size_t)attn_ds_blocks(L) * 2048;
}
// Unnormalised block state (m, l, acc) of attention over keys [k_lo, k_hi).
hipError_t attn_block(int dtype, const AttnArgs& a, hipStream_t s);
// state (m, l, acc) := merge(state, state2) (in place); rows [B*L], heads h_q.
hipError_t attn_state_merge(int B, int L, int h_q, int d_h, float* m, float* l, float* acc,
                            const float* m2, const float* l2, const float* acc2,
                            hipStream_t s);
// o = acc / l (dtype, row stride ldo), lse = m + log l.
hipError_t attn_state_finish(int dtype, int B, int L, int h_q, int d_h, const float* m,
                             const float* l, const float* acc, void* o, int64_t ldo,
                             float* lse, hipStream_t s);

}  // namespace q3l
