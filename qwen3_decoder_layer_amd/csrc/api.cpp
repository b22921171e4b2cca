// Host side of the C ABI declared in include/q3layer.h: argument validation,
// the layout of the saved tensors and of the workspace, and the launch
// sequence of the layer's forward (walkthrough page, Steps 1-10) and
// backward (the same steps' adjoints in reverse order).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <atomic>
#include <cstring>
#include <string>

#include "../../include/q3layer.h"
#include "ops.h"

namespace q3l {
namespace {

thread_local std::string g_err;

q3l_status fail(q3l_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
q3l_status fail(q3l_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

#define Q3L_HIP(call)                                                        \
  do {                                                                       \
    const hipError_t e_ = (call);                                            \
    if (e_ != hipSuccess)                                                    \
      return fail(Q3L_EHIP, "%s failed: %s", #call, hipGetErrorString(e_));  \
  } while (0)

constexpr size_t kAlign = 256;
size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Dims {
  int64_t T;
  int d, hq, hkv, dh, ffn, B, L, qd, kvd, nqkv, nqk;
  size_t es;  // element size of cfg.dtype
};

Dims dims_of(const q3l_layer_cfg& c) {
  Dims m{};
  m.B = c.B; m.L = c.L; m.T = (int64_t)c.B * c.L;
  m.d = c.d; m.hq = c.h_q; m.hkv = c.h_kv; m.dh = c.d_h; m.ffn = c.d_ffn;
  m.qd = c.h_q * c.d_h; m.kvd = c.h_kv * c.d_h;
  m.nqkv = m.qd + 2 * m.kvd; m.nqk = m.qd + m.kvd;
  m.es = c.dtype == Q3L_BF16 ? 2 : 4;
  return m;
}

q3l_status validate(const q3l_layer_cfg* c) {
  if (!c) return fail(Q3L_EINVAL, "cfg is NULL");
  if (c->dtype != Q3L_F32 && c->dtype != Q3L_BF16)
    return fail(Q3L_EINVAL, "dtype %d is neither Q3L_F32 nor Q3L_BF16", c->dtype);
  if (c->d <= 0 || c->h_q <= 0 || c->h_kv <= 0 || c->d_h <= 0 || c->d_ffn <= 0 ||
      c->B <= 0 || c->L <= 0)
    return fail(Q3L_EINVAL, "sizes must be positive (d=%d h_q=%d h_kv=%d d_h=%d "
                "d_ffn=%d B=%d L=%d)", c->d, c->h_q, c->h_kv, c->d_h, c->d_ffn,
                c->B, c->L);
  if (c->h_q % c->h_kv != 0)
    return fail(Q3L_EINVAL, "h_q=%d is not a multiple of h_kv=%d", c->h_q, c->h_kv);
  if (c->d_h != 64 && c->d_h != 128)
    return fail(Q3L_EUNSUPPORTED, "d_h=%d: only 64 and 128 are supported", c->d_h);
  if (c->d % 8 != 0 || c->d_ffn % 8 != 0)
    return fail(Q3L_EUNSUPPORTED, "d=%d and d_ffn=%d must be multiples of 8", c->d,
                c->d_ffn);
  if (c->d > 8192)
    return fail(Q3L_EUNSUPPORTED, "d=%d exceeds 8192", c->d);
  if (!(c->eps > 0.0f) || !std::isfinite(c->eps))
    return fail(Q3L_EINVAL, "eps must be positive and finite");
  if (!(c->rope_theta > 0.0f) || !std::isfinite(c->rope_theta))
    return fail(Q3L_EINVAL, "rope_theta must be positive and finite");
  if ((c->qk_norm != 0 && c->qk_norm != 1) || (c->tp_partial != 0 && c->tp_partial != 1))
    return fail(Q3L_EINVAL, "qk_norm and tp_partial must be 0 or 1");
  const int64_t T = (int64_t)c->B * c->L;
  const int64_t widest = std::max<int64_t>(2LL * c->d_ffn,
                                           (int64_t)(c->h_q + 2 * c->h_kv) * c->d_h);
  if (T > (1LL << 30) || widest > (1LL << 30) || (int64_t)c->h_q * c->d_h > (1LL << 30))
    return fail(Q3L_EUNSUPPORTED, "sizes exceed the 32-bit index range");
  if (c->L > 65535LL * 32)
    return fail(Q3L_EUNSUPPORTED, "L=%d too long", c->L);
  // The bf16 GEMM addresses each operand with 32-bit byte offsets.
  if (c->dtype == Q3L_BF16) {
    const int64_t widest_act = std::max<int64_t>(widest, (int64_t)c->d);
    if ((T + 8) * widest_act * 2 >= (1LL << 31))
      return fail(Q3L_EUNSUPPORTED, "B*L=%lld tokens x %lld features exceeds 2 GiB per "
                  "activation tensor", (long long)T, (long long)widest_act);
    const int64_t wmax = std::max<int64_t>((int64_t)c->d_ffn,
                                           (int64_t)(c->h_q + 2 * c->h_kv) * c->d_h);
    if ((wmax + 8) * c->d * 2 >= (1LL << 31))
      return fail(Q3L_EUNSUPPORTED, "a %lld x %d weight exceeds 2 GiB", (long long)wmax,
                  c->d);
  }
  return Q3L_OK;
}

// The backward's transposed copies exist only for a bf16 layer with a
// backward (not for the forward-only tensor-parallel share).
bool has_transposes(const q3l_layer_cfg& c) { return c.dtype == Q3L_BF16 && !c.tp_partial; }

q3l_saved_layout saved_layout(const q3l_layer_cfg& c) {
  const Dims m = dims_of(c);
  q3l_saved_layout s{};
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += up(bytes); return o; };
  s.rstd1 = take(m.T * 4);
  s.xn = take(m.T * m.d * m.es);
  s.qkv = take(m.T * m.nqkv * m.es);
  s.qk_rope = take(m.T * m.nqk * m.es);
  s.rstd_q = take(m.T * m.hq * 4);
  s.rstd_k = take(m.T * m.hkv * 4);
  s.rope_cos = take((size_t)m.L * (m.dh / 2) * 4);
  s.rope_sin = take((size_t)m.L * (m.dh / 2) * 4);
  s.attn_o = take(m.T * m.qd * m.es);
  s.lse = take((size_t)m.B * m.hq * m.L * 4);
  s.h = take(m.T * m.d * m.es);
  s.rstd2 = take(m.T * 4);
  s.hn = take(m.T * m.d * m.es);
  s.gu = take(m.T * 2 * (size_t)m.ffn * m.es);
  s.f = take(m.T * (size_t)m.ffn * m.es);
  // The transposed copy for the backward (bf16): xn^T.  (wt, once the
  // transposed weights, is empty: the input-gradient GEMMs read the weights
  // with transposing LDS loads.)
  s.wt = off;
  s.xnt = off;
  if (has_transposes(c)) take((size_t)m.d * ((m.T + 7) / 8 * 8) * 2);
  s.total = off;
  return s;
}

constexpr size_t kStoredDsMax = size_t(8) << 30;   // the stored-dS workspace cap
constexpr size_t kNone = ~size_t(0);                // no such region

struct BwdWs {
  // wpart_post / wpart_in: partial-row sums of the two RMSNorm weight
  // gradients (separate, so an input-gradient-only call leaves both for the
  // weight-gradient call that follows it).
  size_t dgu, dhn, dh, dO, delta, dqk, dqkv, dxn, wpart_post, wpart_in, qpart, kpart;
  // bf16 only: two scratch buffers for the transposed operands of the
  // weight-gradient GEMMs ([features, Tp]): [dg du]^T, then [dq dk dv]^T
  // (tA), and dy^T (tC); and the attention backward's dS blocks (ds).
  size_t tA, tC, ds;
  size_t total;
};

int64_t pad8(int64_t v) { return (v + 7) / 8 * 8; }

BwdWs bwd_layout(const q3l_layer_cfg& c) {
  const Dims m = dims_of(c);
  BwdWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += up(bytes); return o; };
  w.dgu = take(m.T * 2 * (size_t)m.ffn * m.es);
  w.dhn = take(m.T * m.d * m.es);
  w.dh = take(m.T * m.d * m.es);
  w.dO = take(m.T * m.qd * m.es);
  w.delta = take((size_t)m.B * m.hq * m.L * 4);
  w.dqk = take(m.T * m.nqk * m.es);
  w.dqkv = take(m.T * m.nqkv * m.es);
  w.dxn = take(m.T * m.d * m.es);
  w.wpart_post = take((size_t)rmsnorm_bwd_max_parts() * m.d * 4);
  w.wpart_in = take((size_t)rmsnorm_bwd_max_parts() * m.d * 4);
  w.qpart = take((size_t)qknorm_bwd_max_parts() * m.dh * 4);
  w.kpart = take((size_t)qknorm_bwd_max_parts() * m.dh * 4);
  if (c.dtype == Q3L_BF16) {
    const size_t Tp = (size_t)pad8(m.T);
    w.tA = take((size_t)std::max<int64_t>(std::max<int64_t>(2LL * m.ffn, m.nqkv), m.d) * Tp * 2);
    w.tC = take((size_t)m.d * Tp * 2);
    // dS for the attention backward while it stays within kStoredDsMax
    // (about B h_q L^2 bytes; beyond, the backward recomputes S and dP for dQ).
    w.ds = attn_ds_bytes(m.B, m.L, m.hq) <= kStoredDsMax ? take(attn_ds_bytes(m.B, m.L, m.hq))
                                                         : kNone;
  }
  w.total = off;
  return w;
}

inline char* at(void* base, size_t off) { return static_cast<char*>(base) + off; }
inline const char* at(const void* base, size_t off) { return static_cast<const char*>(base) + off; }

Operand kop(const void* p, int64_t ld, int rows) {
  Operand o{};
  o.p[0] = p; o.ld[0] = ld; o.nseg = 1; o.rows = rows; o.k_contig = 1;
  return o;
}
Operand rop(const void* p, int64_t ld, int rows) {
  Operand o = kop(p, ld, rows);
  o.k_contig = 0;
  return o;
}
void add_seg(Operand& o, const void* p, int64_t ld, int start) {
  o.p[o.nseg] = p; o.ld[o.nseg] = ld; o.start[o.nseg] = start; ++o.nseg;
}

hipError_t gemm(int dtype, const GemmArgs& g, hipStream_t s) {
  return dtype == Q3L_BF16 ? gemm_bf16(g, s) : gemm_f32(g, s);
}

Epilogue epi_store(void* c, int64_t ldc, const void* r, int64_t ldr) {
  Epilogue e{};
  e.kind = EPI_STORE; e.c = c; e.ldc = ldc; e.r = r; e.ldr = ldr;
  return e;
}
Epilogue epi_wgrad(float* c, int64_t ldc, int accumulate) {
  Epilogue e{};
  e.kind = EPI_WGRAD; e.cs[0] = c; e.cnseg = 1; e.ldc = ldc; e.accumulate = accumulate;
  return e;
}

// g = a gate^T, u = a up^T over interleaved 32-row blocks of gate and up,
// epilogue f = silu(g) * u (and g | u into gu when gu != NULL).
GemmArgs swiglu_args(const void* a, int K, int M, const void* gate, const void* up,
                     int ffn, void* f, void* gu) {
  GemmArgs g{};
  g.a = kop(a, K, M);
  g.b = kop(gate, K, ffn);
  add_seg(g.b, up, K, 0);
  g.b.paired = 1;
  g.M = M; g.N = 2 * ((ffn + 31) / 32 * 32); g.K = K;
  g.epi.kind = EPI_SILU_MUL;
  g.epi.c = f; g.epi.ldc = ffn; g.epi.ffn = ffn;
  g.epi.gu = gu; g.epi.ldgu = 2 * (int64_t)ffn;
  return g;
}

#define Q3L_CHECK_PTR(p, name)                                                   \
  do {                                                                           \
    if (!(p)) return fail(Q3L_EINVAL, "%s is NULL", name);                       \
    if (!aligned16(p)) return fail(Q3L_EALIGN, "%s is not 16-byte aligned", name); \
  } while (0)

q3l_status check_weights(const q3l_weights* w, bool need_qk) {
  if (!w) return fail(Q3L_EINVAL, "weights struct is NULL");
  Q3L_CHECK_PTR(w->in_norm, "w.in_norm");
  Q3L_CHECK_PTR(w->q, "w.q");
  Q3L_CHECK_PTR(w->k, "w.k");
  Q3L_CHECK_PTR(w->v, "w.v");
  if (need_qk) {
    Q3L_CHECK_PTR(w->q_norm, "w.q_norm");
    Q3L_CHECK_PTR(w->k_norm, "w.k_norm");
  }
  Q3L_CHECK_PTR(w->o, "w.o");
  Q3L_CHECK_PTR(w->post_norm, "w.post_norm");
  Q3L_CHECK_PTR(w->gate, "w.gate");
  Q3L_CHECK_PTR(w->up, "w.up");
  Q3L_CHECK_PTR(w->down, "w.down");
  return Q3L_OK;
}

// ---- phases and their marks --------------------------------------------
// The steps of a forward / backward call in launch order.  With marks, the
// call records event 0 before its first kernel and event i + 1 after phase
// i (an empty phase records its event right after the previous one).
const char* const kFwdPhases[] = {
    "F1 rmsnorm",
    "F2 qkv gemm",
    "F3-F4 qk-norm + rope",
    "transposes for the backward",
    "F5 attention",
    "F6 o gemm + residual",
    "F7 rmsnorm",
    "F8-F9 gate/up gemm + swiglu",
    "F10 down gemm + residual",
};
const char* const kBwdPhases[] = {
    "B1 down dgrad gemm",
    "B2 swiglu adjoint",
    "B1 down wgrad transposes",
    "B1 down wgrad gemm",
    "B3 gate/up dgrad gemm",
    "B3 gate/up wgrad transposes",
    "B3 gate/up wgrad gemm",
    "B4 rmsnorm bwd",
    "B5 o dgrad gemm",
    "B5 o wgrad transposes",
    "B5 o wgrad gemm",
    "B6 attention bwd",
    "B7 qk-norm + rope bwd",
    "B8 qkv dgrad gemm",
    "B8 qkv wgrad transposes",
    "B8 qkv wgrad gemm",
    "B9 rmsnorm bwd",
};
constexpr int kNumFwdPhases = sizeof(kFwdPhases) / sizeof(kFwdPhases[0]);
constexpr int kNumBwdPhases = sizeof(kBwdPhases) / sizeof(kBwdPhases[0]);

// Orders the caller's stream after work forked to its second stream: on
// the way out of the call, whatever path it takes, the caller's stream waits
// for the join event (join() does it early and reports the status).
struct Join {
  hipStream_t s = nullptr;
  hipEvent_t ev = nullptr;
  hipError_t join() {
    const hipError_t e = ev ? hipStreamWaitEvent(s, ev, 0) : hipSuccess;
    ev = nullptr;
    return e;
  }
  ~Join() { (void)join(); }
};

struct Marks {
  void* const* ev = nullptr;
  int next = 0;
  hipStream_t s = nullptr;
  // Records the mark that ends phase `phase` (and any skipped before it).
  hipError_t end(int phase) {
    if (!ev) return hipSuccess;
    while (next <= phase + 1) {
      const hipError_t e = hipEventRecord(static_cast<hipEvent_t>(ev[next++]), s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
};

q3l_status check_exec(const q3l_exec* ex, int nphases, bool uses_side) {
  if (!ex) return Q3L_OK;
  if (ex->marks) {
    if (ex->n_marks != nphases + 1)
      return fail(Q3L_EINVAL, "exec.n_marks is %d, this call records %d marks", ex->n_marks,
                  nphases + 1);
    for (int i = 0; i <= nphases; ++i)
      if (!ex->marks[i]) return fail(Q3L_EINVAL, "exec.marks[%d] is NULL", i);
  } else if (ex->n_marks != 0) {
    return fail(Q3L_EINVAL, "exec.n_marks is %d but exec.marks is NULL", ex->n_marks);
  }
  if (uses_side && ex->side_stream && (!ex->fork_event || !ex->join_event))
    return fail(Q3L_EINVAL, "exec.side_stream needs exec.fork_event and exec.join_event");
  return Q3L_OK;
}

}  // namespace
}  // namespace q3l

using namespace q3l;

extern "C" {

const char* q3l_last_error(void) { return g_err.c_str(); }
int q3l_version(void) { return Q3L_VERSION; }

int q3l_phase_count(int backward) { return backward ? kNumBwdPhases : kNumFwdPhases; }
const char* q3l_phase_name(int backward, int i) {
  if (i < 0 || i >= q3l_phase_count(backward)) return nullptr;
  return backward ? kBwdPhases[i] : kFwdPhases[i];
}

q3l_status q3l_validate(const q3l_layer_cfg* cfg) {
  const q3l_status st = validate(cfg);
  if (st == Q3L_OK) g_err.clear();
  return st;
}

q3l_status q3l_saved_layout_of(const q3l_layer_cfg* cfg, q3l_saved_layout* out) {
  const q3l_status st = validate(cfg);
  if (st != Q3L_OK) return st;
  if (!out) return fail(Q3L_EINVAL, "out is NULL");
  *out = saved_layout(*cfg);
  return Q3L_OK;
}

// The copy the bf16 backward reads in K-contiguous form, from an input the
// forward already has: xn^T [d, Tp] (the QKV weight gradient's second
// operand), columns >= T zero.
hipError_t transposed_copies(const q3l_layer_cfg& c, const void* xn, char* xnt, hipStream_t s) {
  const Dims m = dims_of(c);
  const int d = m.d;
  const int T = (int)m.T, Tp = (int)((m.T + 7) / 8 * 8);
  const TransposeJob jobs[1] = {{xn, d, xnt, Tp, T, Tp, d}};
  return transpose_bf16_batch(jobs, 1, s);
}

size_t q3l_saved_bytes(const q3l_layer_cfg* cfg) {
  if (validate(cfg) != Q3L_OK) return 0;
  return saved_layout(*cfg).total;
}

size_t q3l_workspace_bytes(const q3l_layer_cfg* cfg, int backward) {
  if (validate(cfg) != Q3L_OK) return 0;
  // Forward without `saved`: room for the intermediates up to (not
  // including) the backward's transposed copies.
  return backward ? bwd_layout(*cfg).total : saved_layout(*cfg).wt;
}

q3l_status q3l_layer_forward(const q3l_layer_cfg* cfg, const q3l_weights* w,
                             const void* x, const q3l_outputs* out, void* saved,
                             void* workspace, size_t workspace_bytes, void* stream,
                             const q3l_exec* exec) {
  q3l_status st = validate(cfg);
  if (st != Q3L_OK) return st;
  const q3l_layer_cfg& c = *cfg;
  if ((st = check_weights(w, c.qk_norm != 0)) != Q3L_OK) return st;
  Q3L_CHECK_PTR(x, "x");
  if (!out) return fail(Q3L_EINVAL, "out is NULL");
  if (c.tp_partial) {
    Q3L_CHECK_PTR(out->attn_partial, "out.attn_partial");
    Q3L_CHECK_PTR(out->mlp_partial, "out.mlp_partial");
  } else {
    Q3L_CHECK_PTR(out->y, "out.y");
  }
  const q3l_saved_layout L = saved_layout(c);
  void* S = saved;
  if (S) {
    Q3L_CHECK_PTR(S, "saved");
  } else {
    Q3L_CHECK_PTR(workspace, "workspace");
    if (workspace_bytes < L.wt)
      return fail(Q3L_EINVAL, "workspace holds %zu bytes, %zu needed", workspace_bytes,
                  L.wt);
    S = workspace;
  }
  const bool copies = saved && has_transposes(c);
  if ((st = check_exec(exec, kNumFwdPhases, copies)) != Q3L_OK) return st;
  const Dims m = dims_of(c);
  const int dt = c.dtype;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Marks mk;
  mk.s = s;
  mk.ev = exec ? exec->marks : nullptr;
  hipStream_t side = (copies && exec) ? static_cast<hipStream_t>(exec->side_stream) : nullptr;
  Join joiner;
  float* rstd1 = reinterpret_cast<float*>(at(S, L.rstd1));
  void* xn = at(S, L.xn);
  void* qkv = at(S, L.qkv);
  void* qkr = at(S, L.qk_rope);
  float* rq = reinterpret_cast<float*>(at(S, L.rstd_q));
  float* rk = reinterpret_cast<float*>(at(S, L.rstd_k));
  float* cs = reinterpret_cast<float*>(at(S, L.rope_cos));
  float* sn = reinterpret_cast<float*>(at(S, L.rope_sin));
  void* ao = at(S, L.attn_o);
  float* lse = reinterpret_cast<float*>(at(S, L.lse));
  void* h = at(S, L.h);
  float* rstd2 = reinterpret_cast<float*>(at(S, L.rstd2));
  void* hn = at(S, L.hn);
  void* gu = at(S, L.gu);
  void* f = at(S, L.f);
  const char* qkvp = static_cast<const char*>(qkv);

  Q3L_HIP(mk.end(-1));
  // Step 1: input RMSNorm.
  Q3L_HIP(rmsnorm_fwd(dt, m.T, m.d, x, w->in_norm, c.eps, xn, rstd1, s));
  Q3L_HIP(mk.end(0));
  // Step 2: q/k/v projections as one GEMM over the stacked weights.
  {
    GemmArgs g{};
    g.a = kop(xn, m.d, (int)m.T);
    g.b = kop(w->q, m.d, m.nqkv);
    add_seg(g.b, w->k, m.d, m.qd);
    add_seg(g.b, w->v, m.d, m.qd + m.kvd);
    g.M = (int)m.T; g.N = m.nqkv; g.K = m.d;
    g.epi = epi_store(qkv, m.nqkv, nullptr, 0);
    Q3L_HIP(gemm(dt, g, s));
  }
  Q3L_HIP(mk.end(1));
  // Steps 3-4: per-head q/k RMSNorm, then RoPE.
  Q3L_HIP(rope_table(m.L, m.dh, c.rope_theta, cs, sn, s));
  Q3L_HIP(qknorm_rope_fwd(dt, m.B, m.L, m.hq, m.hkv, m.dh, c.qk_norm, c.eps, qkv,
                          m.nqkv, w->q_norm, w->k_norm, cs, sn, qkr, m.nqk, rq, rk, s));
  Q3L_HIP(mk.end(2));
  // The backward's transposed copies: on the caller's stream here, or on the
  // caller's second stream beside the attention step.
  if (copies && !side) Q3L_HIP(transposed_copies(c, xn, at(S, L.xnt), s));
  Q3L_HIP(mk.end(3));
  // Step 5: causal GQA attention.
  {
    AttnArgs a{};
    a.B = m.B; a.L = m.L; a.h_q = m.hq; a.h_kv = m.hkv; a.d_h = m.dh;
    a.q = qkr; a.ldq = m.nqk;
    a.k = static_cast<const char*>(qkr) + (size_t)m.qd * m.es; a.ldk = m.nqk;
    a.v = qkvp + (size_t)(m.qd + m.kvd) * m.es; a.ldv = m.nqkv;
    a.o = ao; a.ldo = m.qd; a.lse = lse;
    if (side) {
      hipEvent_t fork = static_cast<hipEvent_t>(exec->fork_event);
      hipEvent_t join = static_cast<hipEvent_t>(exec->join_event);
      Q3L_HIP(hipEventRecord(fork, s));
      Q3L_HIP(hipStreamWaitEvent(side, fork, 0));
      const hipError_t e1 = transposed_copies(c, xn, at(S, L.xnt), side);
      const hipError_t e2 = hipEventRecord(join, side);
      // The caller's stream waits for the join at the end of the forward
      // (on any path out of it: `joiner`), not here, so the attention's
      // phase holds no cross-stream wait.
      if (e2 == hipSuccess) { joiner.s = s; joiner.ev = join; }
      const hipError_t e3 = attn_fwd(dt, a, s);
      Q3L_HIP(e1);
      Q3L_HIP(e2);
      Q3L_HIP(e3);
    } else {
      Q3L_HIP(attn_fwd(dt, a, s));
    }
  }
  Q3L_HIP(mk.end(4));
  // Steps 6-7: o_proj with the residual in the epilogue.
  {
    GemmArgs g{};
    g.a = kop(ao, m.qd, (int)m.T);
    g.b = kop(w->o, m.qd, m.d);
    g.M = (int)m.T; g.N = m.d; g.K = m.qd;
    if (c.tp_partial) {
      g.epi.kind = EPI_PARTIAL;
      g.epi.p32 = out->attn_partial; g.epi.ldp = m.d;
      g.epi.c = h; g.epi.ldc = m.d; g.epi.r = x; g.epi.ldr = m.d;
    } else {
      g.epi = epi_store(h, m.d, x, m.d);
    }
    Q3L_HIP(gemm(dt, g, s));
  }
  Q3L_HIP(mk.end(5));
  // Step 8: post-attention RMSNorm.
  Q3L_HIP(rmsnorm_fwd(dt, m.T, m.d, h, w->post_norm, c.eps, hn, rstd2, s));
  Q3L_HIP(mk.end(6));
  // Step 9: gate/up as one GEMM over interleaved rows, silu(g) * u fused.
  Q3L_HIP(gemm(dt, swiglu_args(hn, m.d, (int)m.T, w->gate, w->up, m.ffn, f,
                               saved ? gu : nullptr), s));
  Q3L_HIP(mk.end(7));
  // Steps 9-10: down projection with the residual in the epilogue.
  {
    GemmArgs g{};
    g.a = kop(f, m.ffn, (int)m.T);
    g.b = kop(w->down, m.ffn, m.d);
    g.M = (int)m.T; g.N = m.d; g.K = m.ffn;
    if (c.tp_partial) {
      g.epi.kind = EPI_PARTIAL;
      g.epi.p32 = out->mlp_partial; g.epi.ldp = m.d;
    } else {
      g.epi = epi_store(out->y, m.d, h, m.d);
    }
    Q3L_HIP(gemm(dt, g, s));
  }
  Q3L_HIP(mk.end(8));
  Q3L_HIP(joiner.join());
  g_err.clear();
  return Q3L_OK;
}

q3l_status q3l_layer_backward(const q3l_layer_cfg* cfg, const q3l_weights* w,
                              const void* x, const void* dy, const void* saved,
                              void* dx, const q3l_grads* grads, int flags,
                              void* workspace, size_t workspace_bytes, void* stream,
                              const q3l_exec* exec) {
  q3l_status st = validate(cfg);
  if (st != Q3L_OK) return st;
  const q3l_layer_cfg& c = *cfg;
  if (c.tp_partial)
    return fail(Q3L_EUNSUPPORTED, "backward of a tp_partial layer is not provided");
  if ((st = check_weights(w, c.qk_norm != 0)) != Q3L_OK) return st;
  if (flags & ~(Q3L_BWD_INPUT | Q3L_BWD_WEIGHT | Q3L_BWD_ACCUMULATE | Q3L_BWD_DEFERRED_WEIGHT))
    return fail(Q3L_EINVAL, "unknown flag bits 0x%x", flags);
  const bool want_dx = flags & Q3L_BWD_INPUT, want_w = flags & Q3L_BWD_WEIGHT;
  const bool deferred = flags & Q3L_BWD_DEFERRED_WEIGHT;
  if (deferred && (!want_w || want_dx))
    return fail(Q3L_EINVAL, "Q3L_BWD_DEFERRED_WEIGHT goes with Q3L_BWD_WEIGHT and "
                "without Q3L_BWD_INPUT");
  // The input-gradient chain runs unless a previous INPUT-only call on this
  // workspace already ran it.
  const bool chain = !deferred;
  const int acc = (flags & Q3L_BWD_ACCUMULATE) ? 1 : 0;
  Q3L_CHECK_PTR(x, "x");
  Q3L_CHECK_PTR(dy, "dy");
  Q3L_CHECK_PTR(saved, "saved");
  Q3L_CHECK_PTR(workspace, "workspace");
  if (want_dx) Q3L_CHECK_PTR(dx, "dx");
  if (want_w) {
    if (!grads) return fail(Q3L_EINVAL, "grads struct is NULL");
    Q3L_CHECK_PTR(grads->in_norm, "grads.in_norm");
    Q3L_CHECK_PTR(grads->q, "grads.q");
    Q3L_CHECK_PTR(grads->k, "grads.k");
    Q3L_CHECK_PTR(grads->v, "grads.v");
    if (c.qk_norm) {
      Q3L_CHECK_PTR(grads->q_norm, "grads.q_norm");
      Q3L_CHECK_PTR(grads->k_norm, "grads.k_norm");
    }
    Q3L_CHECK_PTR(grads->o, "grads.o");
    Q3L_CHECK_PTR(grads->post_norm, "grads.post_norm");
    Q3L_CHECK_PTR(grads->gate, "grads.gate");
    Q3L_CHECK_PTR(grads->up, "grads.up");
    Q3L_CHECK_PTR(grads->down, "grads.down");
  }
  const BwdWs W = bwd_layout(c);
  if (workspace_bytes < W.total)
    return fail(Q3L_EINVAL, "workspace holds %zu bytes, %zu needed", workspace_bytes,
                W.total);
  if ((st = check_exec(exec, kNumBwdPhases, false)) != Q3L_OK) return st;

  const q3l_saved_layout L = saved_layout(c);
  const Dims m = dims_of(c);
  const int dt = c.dtype;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Marks mk;
  mk.s = s;
  mk.ev = exec ? exec->marks : nullptr;
  Q3L_HIP(mk.end(-1));
  if (!want_dx && !want_w) {
    Q3L_HIP(mk.end(kNumBwdPhases - 1));
    g_err.clear();
    return Q3L_OK;
  }
  const float* rstd1 = reinterpret_cast<const float*>(at(saved, L.rstd1));
  const void* xn = at(saved, L.xn);
  const char* qkv = at(saved, L.qkv);
  const char* qkr = at(saved, L.qk_rope);
  const float* rq = reinterpret_cast<const float*>(at(saved, L.rstd_q));
  const float* rk = reinterpret_cast<const float*>(at(saved, L.rstd_k));
  const float* cs = reinterpret_cast<const float*>(at(saved, L.rope_cos));
  const float* sn = reinterpret_cast<const float*>(at(saved, L.rope_sin));
  const void* ao = at(saved, L.attn_o);
  const float* lse = reinterpret_cast<const float*>(at(saved, L.lse));
  const void* h = at(saved, L.h);
  const float* rstd2 = reinterpret_cast<const float*>(at(saved, L.rstd2));
  const void* hn = at(saved, L.hn);
  const void* gu = at(saved, L.gu);
  const void* f = at(saved, L.f);
  void* dgu = at(workspace, W.dgu);
  void* dhn = at(workspace, W.dhn);
  void* dh = at(workspace, W.dh);
  void* dO = at(workspace, W.dO);
  float* delta = reinterpret_cast<float*>(at(workspace, W.delta));
  char* dqk = at(workspace, W.dqk);
  char* dqkv = at(workspace, W.dqkv);
  void* dxn = at(workspace, W.dxn);
  float* wpart_post = reinterpret_cast<float*>(at(workspace, W.wpart_post));
  float* wpart_in = reinterpret_cast<float*>(at(workspace, W.wpart_in));
  float* qpart = reinterpret_cast<float*>(at(workspace, W.qpart));
  float* kpart = reinterpret_cast<float*>(at(workspace, W.kpart));
  const int T = (int)m.T;
  // Partial-row counts of the norm-weight reductions: fixed by the shapes,
  // so a deferred weight-gradient call knows them without the chain.
  const int np_norm = rmsnorm_bwd_parts(dt, m.T, m.d);
  const int np_qk = qknorm_bwd_parts(m.T, m.hq + m.hkv, m.dh);

  // bf16: the input-gradient GEMMs read the weights [out, in] as they are,
  // with the matrix-core kernel's transposing LDS loads (as fast as a
  // transposed copy for all but the down projection, and no copy to write).
  // The weight-gradient GEMMs contract over the tokens and run in the
  // K-contiguous form: xn^T comes from the saved block (the forward wrote
  // it), their other operands are transposed to [features, T] (T padded to
  // a multiple of 8 with zeros) into reused scratch buffers.
  const bool bt = dt == Q3L_BF16;
  const int Tp = (int)pad8(m.T);
  const char* xnt = bt ? at(saved, L.xnt) : nullptr;
  char* tA = bt ? at(workspace, W.tA) : nullptr;
  char* tC = bt ? at(workspace, W.tC) : nullptr;
  // Weight gradient dW[ma, nb] (+)= sum_t A[t, ma] B[t, nb] (ma, nb are
  // feature counts; A/B activations with row strides lda/ldb), as two
  // phases: the operand transposes (bf16; one launch, skipping those marked
  // done) and the GEMM.  Forms (bf16; the fp32 path reads both in place):
  //   kCopies  both operands transposed to [features, Tp] copies, read
  //            K-contiguous (32x32x16 instructions);
  //   kACopy   A transposed, B read in place with the transposing LDS loads
  //            (the input-gradient form, 16x16x32 instructions);
  //   kInPlace both read in place.
  // Measured on the layer's shapes: kACopy is 2-5% faster than kCopies for
  // the down and gate/up gradients and saves B's copy, kCopies is 10% faster
  // for the QKV gradient (its 192-row tiles fill the CUs), and kInPlace
  // matches kCopies for the o gradient without any copy.
  enum WForm { kCopies, kACopy, kInPlace };
  auto wgrad = [&](int phase_t, const void* A, int lda, int ma, const void* B, int ldb,
                   int nb, Epilogue e, char* ta, char* tb, bool a_done,
                   bool b_done, WForm form) -> hipError_t {
    GemmArgs g{};
    if (bt && form != kInPlace) {
      TransposeJob jobs[2];
      int nj = 0;
      if (!a_done) jobs[nj++] = TransposeJob{A, lda, ta, Tp, T, Tp, ma};
      if (form == kCopies && !b_done) jobs[nj++] = TransposeJob{B, ldb, tb, Tp, T, Tp, nb};
      hipError_t err = transpose_bf16_batch(jobs, nj, s);
      if (err != hipSuccess) return err;
      if ((err = mk.end(phase_t)) != hipSuccess) return err;
      g.a = kop(ta, Tp, ma);
      if (form == kCopies) {
        g.b = kop(tb, Tp, nb);
        g.K = Tp;
      } else {
        g.b = rop(B, ldb, nb);
        g.K = T;
      }
    } else {
      const hipError_t err = mk.end(phase_t);
      if (err != hipSuccess) return err;
      g.a = rop(A, lda, ma);
      g.b = rop(B, ldb, nb);
      g.K = T;
    }
    g.M = ma; g.N = nb;
    g.epi = e;
    const hipError_t err = gemm(dt, g, s);
    if (err != hipSuccess) return err;
    return mk.end(phase_t + 1);
  };

  // Step 9 (down_proj): df = dy W_down.  fp32: fused with the SwiGLU adjoint
  // in the GEMM epilogue.  bf16: df lands in the dg half of dgu, and a
  // separate pass turns it into dg | du, writing the transposed copy the
  // gate/up weight gradient reads as well: [dg du]^T (an epilogue that reads
  // g, u would hold the matrix cores idle while it waits on memory).
  if (chain) {
    GemmArgs g{};
    g.a = kop(dy, m.d, T);
    g.b = rop(w->down, m.ffn, m.ffn);
    g.M = T; g.N = m.ffn; g.K = m.d;
    if (bt) {
      g.epi = epi_store(dgu, 2 * (int64_t)m.ffn, nullptr, 0);
    } else {
      g.epi.kind = EPI_SILU_BWD;
      g.epi.c = dgu; g.epi.ldc = 2 * (int64_t)m.ffn;
      g.epi.r = gu; g.epi.ldr = 2 * (int64_t)m.ffn; g.epi.ffn = m.ffn;
    }
    Q3L_HIP(gemm(dt, g, s));
  }
  Q3L_HIP(mk.end(0));
  if (bt && chain)
    Q3L_HIP(swiglu_bwd_bf16(T, Tp, m.ffn, dgu, 2 * (int64_t)m.ffn, gu, 2 * (int64_t)m.ffn,
                            dgu, 2 * (int64_t)m.ffn, want_w ? tA : nullptr, Tp, s));
  if (bt && deferred)   // [dg du]^T from the dg | du the INPUT call left
    Q3L_HIP(swiglu_transposes_bf16(T, Tp, m.ffn, dgu, 2 * (int64_t)m.ffn, tA, Tp, s));
  Q3L_HIP(mk.end(1));
  if (want_w)  // dW_down = dy^T f  (bf16: dy^T into tC, f read in place)
    Q3L_HIP(wgrad(2, dy, m.d, m.d, f, m.ffn, m.ffn, epi_wgrad(grads->down, m.ffn, acc), tC,
                  nullptr, false, false, kACopy));
  Q3L_HIP(mk.end(3));
  // Step 9 (gate/up): dhn = dg W_gate + du W_up (one GEMM over stacked K).
  if (chain) {
    GemmArgs g{};
    g.a = kop(dgu, 2 * (int64_t)m.ffn, T);
    g.b = rop(w->gate, m.d, m.d);
    add_seg(g.b, w->up, m.d, m.ffn);
    g.M = T; g.N = m.d; g.K = 2 * m.ffn;
    g.epi = epi_store(dhn, m.d, nullptr, 0);
    Q3L_HIP(gemm(dt, g, s));
  }
  Q3L_HIP(mk.end(4));
  if (want_w) {  // dW_gate | dW_up = [dg du]^T hn  ([dg du]^T already in tA, hn in place)
    Epilogue e = epi_wgrad(grads->gate, m.d, acc);
    e.cs[1] = grads->up; e.cstart[1] = m.ffn; e.cnseg = 2;
    Q3L_HIP(wgrad(5, dgu, 2 * m.ffn, 2 * m.ffn, hn, m.d, m.d, e, tA, nullptr, bt, false,
                  kACopy));
  }
  Q3L_HIP(mk.end(6));
  // Steps 8 and 10: post-attention RMSNorm adjoint plus the residual dy.
  if (chain) {
    int np = 0;
    Q3L_HIP(rmsnorm_bwd(dt, m.T, m.d, dhn, h, rstd2, w->post_norm, dy, dh, wpart_post, &np, s));
  }
  if (want_w) Q3L_HIP(reduce_rows(wpart_post, np_norm, m.d, grads->post_norm, acc, s));
  Q3L_HIP(mk.end(7));
  // Step 6: dO = dh W_o.
  if (chain) {
    GemmArgs g{};
    g.a = kop(dh, m.d, T);
    g.b = rop(w->o, m.qd, m.qd);
    g.M = T; g.N = m.qd; g.K = m.d;
    g.epi = epi_store(dO, m.qd, nullptr, 0);
    Q3L_HIP(gemm(dt, g, s));
  }
  Q3L_HIP(mk.end(8));
  if (want_w)  // dW_o = dh^T O, both operands read in place
    Q3L_HIP(wgrad(9, dh, m.d, m.d, ao, m.qd, m.qd, epi_wgrad(grads->o, m.qd, acc), nullptr,
                  nullptr, false, false, kInPlace));
  Q3L_HIP(mk.end(10));
  // Step 5: attention backward (P recomputed from the log-sum-exp; bf16:
  // dQ formed from the dS that the dK/dV kernel stores).
  if (chain) {
    AttnArgs a{};
    a.B = m.B; a.L = m.L; a.h_q = m.hq; a.h_kv = m.hkv; a.d_h = m.dh;
    a.q = qkr; a.ldq = m.nqk;
    a.k = qkr + (size_t)m.qd * m.es; a.ldk = m.nqk;
    a.v = qkv + (size_t)(m.qd + m.kvd) * m.es; a.ldv = m.nqkv;
    a.o = const_cast<void*>(ao); a.ldo = m.qd; a.lse = const_cast<float*>(lse);
    a.dout = dO; a.lddo = m.qd;
    a.dq = dqk; a.dk = dqk + (size_t)m.qd * m.es;
    a.dv = dqkv + (size_t)(m.qd + m.kvd) * m.es;
    a.delta = delta;
    a.ds = (bt && W.ds != kNone) ? at(workspace, W.ds) : nullptr;
    Q3L_HIP(attn_bwd(dt, a, s));
  }
  Q3L_HIP(mk.end(11));
  // Steps 4-3: RoPE adjoint and q/k RMSNorm adjoint.
  if (chain) {
    int np = 0;
    Q3L_HIP(qknorm_rope_bwd(dt, m.B, m.L, m.hq, m.hkv, m.dh, c.qk_norm, dqk, m.nqk,
                            qkv, m.nqkv, w->q_norm, w->k_norm, rq, rk, cs, sn, dqkv,
                            m.nqkv, qpart, kpart, &np, s));
  }
  if (want_w && c.qk_norm)
    Q3L_HIP(reduce_rows2(qpart, kpart, np_qk, m.dh, grads->q_norm, grads->k_norm, acc, s));
  Q3L_HIP(mk.end(12));
  // Step 2: dxn = [dq dk dv] [W_q; W_k; W_v].
  if (chain) {
    GemmArgs g{};
    g.a = kop(dqkv, m.nqkv, T);
    g.b = rop(w->q, m.d, m.d);
    add_seg(g.b, w->k, m.d, m.qd);
    add_seg(g.b, w->v, m.d, m.qd + m.kvd);
    g.M = T; g.N = m.d; g.K = m.nqkv;
    g.epi = epi_store(dxn, m.d, nullptr, 0);
    Q3L_HIP(gemm(dt, g, s));
  }
  Q3L_HIP(mk.end(13));
  if (want_w) {  // dW_q | dW_k | dW_v = [dq dk dv]^T xn  (bf16: xn^T saved)
    Epilogue e = epi_wgrad(grads->q, m.d, acc);
    e.cs[1] = grads->k; e.cstart[1] = m.qd;
    e.cs[2] = grads->v; e.cstart[2] = m.qd + m.kvd;
    e.cnseg = 3;
    Q3L_HIP(wgrad(14, dqkv, m.nqkv, m.nqkv, xn, m.d, m.d, e, tA, const_cast<char*>(xnt),
                  false, bt, kCopies));
  }
  Q3L_HIP(mk.end(15));
  // Step 1: input RMSNorm adjoint plus the attention residual dh.
  if (chain) {
    int np = 0;
    Q3L_HIP(rmsnorm_bwd(dt, m.T, m.d, dxn, x, rstd1, w->in_norm, dh,
                        want_dx ? dx : nullptr, wpart_in, &np, s));
  }
  if (want_w) Q3L_HIP(reduce_rows(wpart_in, np_norm, m.d, grads->in_norm, acc, s));
  Q3L_HIP(mk.end(16));
  g_err.clear();
  return Q3L_OK;
}

// ---------------------------------------------------------------------------
// Phase-level entry points.
// ---------------------------------------------------------------------------
q3l_status q3l_rmsnorm_fwd(int32_t dtype, int64_t rows, int32_t n, const void* x,
                           const void* w, float eps, void* y, float* rstd,
                           void* stream) {
  if (dtype != Q3L_F32 && dtype != Q3L_BF16) return fail(Q3L_EINVAL, "bad dtype");
  if (rows < 0 || n <= 0 || n % 8 != 0) return fail(Q3L_EINVAL, "n must be a positive multiple of 8");
  if (n > 8192) return fail(Q3L_EUNSUPPORTED, "n=%d exceeds 8192", n);
  Q3L_CHECK_PTR(x, "x"); Q3L_CHECK_PTR(w, "w"); Q3L_CHECK_PTR(y, "y"); Q3L_CHECK_PTR(rstd, "rstd");
  Q3L_HIP(rmsnorm_fwd(dtype, rows, n, x, w, eps, y, rstd, static_cast<hipStream_t>(stream)));
  return Q3L_OK;
}

size_t q3l_rmsnorm_bwd_workspace_bytes(int32_t n) {
  if (n <= 0) return 0;
  return up((size_t)rmsnorm_bwd_max_parts() * n * 4);
}

q3l_status q3l_rmsnorm_bwd(int32_t dtype, int64_t rows, int32_t n, const void* dy,
                           const void* x, const float* rstd, const void* w, const void* resid,
                           void* dx, float* dw, int accumulate, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (dtype != Q3L_F32 && dtype != Q3L_BF16) return fail(Q3L_EINVAL, "bad dtype");
  if (rows <= 0 || n <= 0 || n % 8 != 0)
    return fail(Q3L_EINVAL, "need rows > 0 and n a positive multiple of 8");
  if (n > 8192) return fail(Q3L_EUNSUPPORTED, "n=%d exceeds 8192", n);
  if (rows > (1LL << 30)) return fail(Q3L_EUNSUPPORTED, "rows exceed 2^30");
  Q3L_CHECK_PTR(dy, "dy"); Q3L_CHECK_PTR(x, "x"); Q3L_CHECK_PTR(rstd, "rstd");
  Q3L_CHECK_PTR(w, "w"); Q3L_CHECK_PTR(dx, "dx"); Q3L_CHECK_PTR(workspace, "workspace");
  if (resid && !aligned16(resid)) return fail(Q3L_EALIGN, "resid is not 16-byte aligned");
  if (dw && !aligned16(dw)) return fail(Q3L_EALIGN, "dw is not 16-byte aligned");
  if (workspace_bytes < q3l_rmsnorm_bwd_workspace_bytes(n))
    return fail(Q3L_EINVAL, "workspace holds %zu bytes, %zu needed", workspace_bytes,
                q3l_rmsnorm_bwd_workspace_bytes(n));
  hipStream_t s = static_cast<hipStream_t>(stream);
  int np = 0;
  float* part = static_cast<float*>(workspace);
  Q3L_HIP(rmsnorm_bwd(dtype, rows, n, dy, x, rstd, w, resid, dx, part, &np, s));
  if (dw) Q3L_HIP(reduce_rows(part, np, n, dw, accumulate ? 1 : 0, s));
  return Q3L_OK;
}

q3l_status q3l_rope_table(int32_t L, int32_t d_h, float theta, float* cos_t, float* sin_t,
                          void* stream) {
  if (L <= 0 || (d_h != 64 && d_h != 128)) return fail(Q3L_EINVAL, "need L > 0, d_h 64 or 128");
  if (!(theta > 0.0f) || !std::isfinite(theta)) return fail(Q3L_EINVAL, "bad theta");
  if ((int64_t)L * d_h > (1LL << 30)) return fail(Q3L_EUNSUPPORTED, "L too long");
  Q3L_CHECK_PTR(cos_t, "cos_t"); Q3L_CHECK_PTR(sin_t, "sin_t");
  Q3L_HIP(rope_table(L, d_h, theta, cos_t, sin_t, static_cast<hipStream_t>(stream)));
  return Q3L_OK;
}

static q3l_status check_heads(int32_t dtype, int32_t B, int32_t L, int32_t h_q, int32_t h_kv,
                              int32_t d_h) {
  if (dtype != Q3L_F32 && dtype != Q3L_BF16) return fail(Q3L_EINVAL, "bad dtype");
  if (B <= 0 || L <= 0 || h_q <= 0 || h_kv <= 0)
    return fail(Q3L_EINVAL, "need positive B, L and heads");
  if (d_h != 64 && d_h != 128) return fail(Q3L_EUNSUPPORTED, "d_h must be 64 or 128");
  if ((int64_t)B * L * (h_q + h_kv) * d_h > (1LL << 40))
    return fail(Q3L_EUNSUPPORTED, "sizes exceed the index range");
  return Q3L_OK;
}

q3l_status q3l_qknorm_rope_fwd(int32_t dtype, int32_t B, int32_t L, int32_t h_q, int32_t h_kv,
                               int32_t d_h, int32_t qk_norm, float eps, const void* in,
                               int64_t ld_in, const void* wq, const void* wk,
                               const float* cos_t, const float* sin_t, void* out,
                               int64_t ld_out, float* rstd_q, float* rstd_k, void* stream) {
  q3l_status st = check_heads(dtype, B, L, h_q, h_kv, d_h);
  if (st != Q3L_OK) return st;
  if (qk_norm != 0 && qk_norm != 1) return fail(Q3L_EINVAL, "qk_norm must be 0 or 1");
  const int64_t w = (int64_t)(h_q + h_kv) * d_h;
  if (ld_in < w || ld_out < w || ld_in % 8 || ld_out % 8)
    return fail(Q3L_EINVAL, "row strides below (h_q + h_kv) * d_h or not multiples of 8");
  Q3L_CHECK_PTR(in, "in"); Q3L_CHECK_PTR(out, "out");
  Q3L_CHECK_PTR(cos_t, "cos_t"); Q3L_CHECK_PTR(sin_t, "sin_t");
  if (qk_norm) {
    if (!(eps > 0.0f) || !std::isfinite(eps)) return fail(Q3L_EINVAL, "bad eps");
    Q3L_CHECK_PTR(wq, "wq"); Q3L_CHECK_PTR(wk, "wk");
    Q3L_CHECK_PTR(rstd_q, "rstd_q"); Q3L_CHECK_PTR(rstd_k, "rstd_k");
  }
  Q3L_HIP(qknorm_rope_fwd(dtype, B, L, h_q, h_kv, d_h, qk_norm, eps, in, ld_in, wq, wk, cos_t,
                          sin_t, out, ld_out, rstd_q, rstd_k, static_cast<hipStream_t>(stream)));
  return Q3L_OK;
}

size_t q3l_qknorm_rope_bwd_workspace_bytes(int32_t d_h) {
  if (d_h != 64 && d_h != 128) return 0;
  return 2 * up((size_t)qknorm_bwd_max_parts() * d_h * 4);
}

q3l_status q3l_qknorm_rope_bwd(int32_t dtype, int32_t B, int32_t L, int32_t h_q, int32_t h_kv,
                               int32_t d_h, int32_t qk_norm, const void* g, int64_t ld_g,
                               const void* pre, int64_t ld_pre, const void* wq,
                               const void* wk, const float* rstd_q, const float* rstd_k,
                               const float* cos_t, const float* sin_t, void* out,
                               int64_t ld_out, float* dwq, float* dwk, int accumulate,
                               void* workspace, size_t workspace_bytes, void* stream) {
  q3l_status st = check_heads(dtype, B, L, h_q, h_kv, d_h);
  if (st != Q3L_OK) return st;
  if (qk_norm != 0 && qk_norm != 1) return fail(Q3L_EINVAL, "qk_norm must be 0 or 1");
  const int64_t w = (int64_t)(h_q + h_kv) * d_h;
  if (ld_g < w || ld_out < w || ld_g % 8 || ld_out % 8 ||
      (qk_norm && (ld_pre < w || ld_pre % 8)))
    return fail(Q3L_EINVAL, "row strides below (h_q + h_kv) * d_h or not multiples of 8");
  Q3L_CHECK_PTR(g, "g"); Q3L_CHECK_PTR(out, "out");
  Q3L_CHECK_PTR(cos_t, "cos_t"); Q3L_CHECK_PTR(sin_t, "sin_t");
  Q3L_CHECK_PTR(workspace, "workspace");
  if (qk_norm) {
    Q3L_CHECK_PTR(pre, "pre");
    Q3L_CHECK_PTR(wq, "wq"); Q3L_CHECK_PTR(wk, "wk");
    Q3L_CHECK_PTR(rstd_q, "rstd_q"); Q3L_CHECK_PTR(rstd_k, "rstd_k");
  }
  if ((dwq == nullptr) != (dwk == nullptr))
    return fail(Q3L_EINVAL, "dwq and dwk are both given or both NULL");
  if ((dwq && !aligned16(dwq)) || (dwk && !aligned16(dwk)))
    return fail(Q3L_EALIGN, "dwq / dwk not 16-byte aligned");
  if (workspace_bytes < q3l_qknorm_rope_bwd_workspace_bytes(d_h))
    return fail(Q3L_EINVAL, "workspace holds %zu bytes, %zu needed", workspace_bytes,
                q3l_qknorm_rope_bwd_workspace_bytes(d_h));
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* qpart = static_cast<float*>(workspace);
  float* kpart = reinterpret_cast<float*>(
      static_cast<char*>(workspace) + up((size_t)qknorm_bwd_max_parts() * d_h * 4));
  int np = 0;
  Q3L_HIP(qknorm_rope_bwd(dtype, B, L, h_q, h_kv, d_h, qk_norm, g, ld_g, pre, ld_pre, wq, wk,
                          rstd_q, rstd_k, cos_t, sin_t, out, ld_out, qpart, kpart, &np, s));
  if (dwq && qk_norm) Q3L_HIP(reduce_rows2(qpart, kpart, np, d_h, dwq, dwk, accumulate ? 1 : 0, s));
  return Q3L_OK;
}

// The bf16 GEMM addresses each operand with 32-bit byte offsets: an [M, N]
// or [M, K] activation and an [N, K] weight must each stay below 2 GiB (with
// the 8 rows of padding the loads may touch).
static q3l_status check_mnk(int32_t dtype, int64_t M, int32_t N, int32_t K) {
  if (dtype != Q3L_F32 && dtype != Q3L_BF16) return fail(Q3L_EINVAL, "bad dtype");
  if (M < 0 || M > (1LL << 30) || N <= 0 || K <= 0 || N % 8 != 0 || K % 8 != 0)
    return fail(Q3L_EINVAL, "need 0 <= M <= 2^30 and N, K positive multiples of 8");
  if (dtype == Q3L_BF16) {
    const int64_t wide = std::max<int64_t>(N, K);
    if ((M + 8) * wide * 2 >= (1LL << 31) || ((int64_t)N + 8) * K * 2 >= (1LL << 31) ||
        ((int64_t)K + 8) * N * 2 >= (1LL << 31))
      return fail(Q3L_EUNSUPPORTED, "M=%lld N=%d K=%d: an operand exceeds the 2 GiB offset "
                  "range of the bf16 GEMM", (long long)M, N, K);
  }
  return Q3L_OK;
}

q3l_status q3l_linear_fwd(int32_t dtype, int64_t M, int32_t N, int32_t K, const void* a,
                          const void* w, const void* resid, void* y, void* stream) {
  q3l_status st = check_mnk(dtype, M, N, K);
  if (st != Q3L_OK) return st;
  Q3L_CHECK_PTR(a, "a"); Q3L_CHECK_PTR(w, "w"); Q3L_CHECK_PTR(y, "y");
  if (resid && !aligned16(resid)) return fail(Q3L_EALIGN, "resid is not 16-byte aligned");
  GemmArgs g{};
  g.a = kop(a, K, (int)M);
  g.b = kop(w, K, N);
  g.M = (int)M; g.N = N; g.K = K;
  g.epi = epi_store(y, N, resid, N);
  Q3L_HIP(gemm(dtype, g, static_cast<hipStream_t>(stream)));
  return Q3L_OK;
}

q3l_status q3l_linear_dgrad(int32_t dtype, int64_t M, int32_t N, int32_t K,
                            const void* dy, const void* w, void* da, void* stream) {
  q3l_status st = check_mnk(dtype, M, N, K);
  if (st != Q3L_OK) return st;
  Q3L_CHECK_PTR(dy, "dy"); Q3L_CHECK_PTR(w, "w"); Q3L_CHECK_PTR(da, "da");
  GemmArgs g{};
  g.a = kop(dy, N, (int)M);
  g.b = rop(w, K, K);
  g.M = (int)M; g.N = K; g.K = N;
  g.epi = epi_store(da, K, nullptr, 0);
  Q3L_HIP(gemm(dtype, g, static_cast<hipStream_t>(stream)));
  return Q3L_OK;
}

q3l_status q3l_linear_wgrad(int32_t dtype, int64_t M, int32_t N, int32_t K,
                            const void* dy, const void* a, float* dw, int accumulate,
                            void* stream) {
  q3l_status st = check_mnk(dtype, M, N, K);
  if (st != Q3L_OK) return st;
  Q3L_CHECK_PTR(dy, "dy"); Q3L_CHECK_PTR(a, "a"); Q3L_CHECK_PTR(dw, "dw");
  if (M == 0) return fail(Q3L_EINVAL, "M must be positive for a weight gradient");
  GemmArgs g{};
  g.a = rop(dy, N, N);
  g.b = rop(a, K, K);
  g.M = N; g.N = K; g.K = (int)M;
  g.epi = epi_wgrad(dw, K, accumulate ? 1 : 0);
  Q3L_HIP(gemm(dtype, g, static_cast<hipStream_t>(stream)));
  return Q3L_OK;
}

q3l_status q3l_swiglu_fwd(int32_t dtype, int64_t M, int32_t N, int32_t K, const void* hn,
                          const void* gate, const void* up, void* f, void* gu,
                          void* stream) {
  // The fused GEMM's logical width is the interleaved gate/up pair, 2 N
  // rounded up to 64 columns; g | u is an [M, 2N] output.
  q3l_status st = check_mnk(dtype, M, N, K);
  if (st == Q3L_OK && N > (1 << 28)) st = fail(Q3L_EUNSUPPORTED, "N=%d too large", N);
  if (st == Q3L_OK) st = check_mnk(dtype, M, 2 * ((N + 31) / 32 * 32), K);
  if (st != Q3L_OK) return st;
  Q3L_CHECK_PTR(hn, "hn"); Q3L_CHECK_PTR(gate, "gate"); Q3L_CHECK_PTR(up, "up");
  Q3L_CHECK_PTR(f, "f");
  if (gu && !aligned16(gu)) return fail(Q3L_EALIGN, "gu is not 16-byte aligned");
  Q3L_HIP(gemm(dtype, swiglu_args(hn, K, (int)M, gate, up, N, f, gu),
               static_cast<hipStream_t>(stream)));
  return Q3L_OK;
}

q3l_status q3l_swiglu_bwd(int32_t dtype, int64_t M, int32_t N, const void* df, const void* gu,
                          void* dgu, void* stream) {
  if (dtype != Q3L_F32 && dtype != Q3L_BF16) return fail(Q3L_EINVAL, "bad dtype");
  if (M < 0 || M > (1LL << 30) - 8 || N <= 0 || N % 8 != 0 || N > (1 << 29))
    return fail(Q3L_EINVAL, "need 0 <= M < 2^30 and N a positive multiple of 8");
  Q3L_CHECK_PTR(df, "df"); Q3L_CHECK_PTR(gu, "gu"); Q3L_CHECK_PTR(dgu, "dgu");
  if (dgu == gu) return fail(Q3L_EINVAL, "dgu may not alias gu");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == Q3L_BF16) {
    Q3L_HIP(swiglu_bwd_bf16((int)M, (int)pad8(M), N, df, N, gu, 2 * (int64_t)N, dgu,
                            2 * (int64_t)N, nullptr, 0, s));
  } else {
    Q3L_HIP(swiglu_bwd_f32(M, N, static_cast<const float*>(df), N,
                           static_cast<const float*>(gu), 2 * (int64_t)N,
                           static_cast<float*>(dgu), 2 * (int64_t)N, s));
  }
  return Q3L_OK;
}

static q3l_status check_attn(int32_t dtype, int32_t B, int32_t L, int32_t h_q, int32_t h_kv,
                             int32_t d_h) {
  if (dtype != Q3L_F32 && dtype != Q3L_BF16) return fail(Q3L_EINVAL, "bad dtype");
  if (B <= 0 || L <= 0 || h_q <= 0 || h_kv <= 0 || h_q % h_kv)
    return fail(Q3L_EINVAL, "need positive B, L, heads and h_q %% h_kv == 0");
  if (d_h != 64 && d_h != 128) return fail(Q3L_EUNSUPPORTED, "d_h must be 64 or 128");
  if (L > 65535LL * 32) return fail(Q3L_EUNSUPPORTED, "L too long");
  return Q3L_OK;
}

// The bf16 attention kernels stage Q/K/V/dO tiles and the per-query
// statistics with 32-bit byte offsets from each tensor's base.
static q3l_status check_attn_range(int32_t dtype, int32_t B, int32_t L, int32_t h_q,
                                   int64_t ld_max) {
  if (dtype != Q3L_BF16) return Q3L_OK;
  const int64_t T = (int64_t)B * L;
  if ((T + 64) * ld_max * 2 >= (1LL << 31) || T * h_q * 4 >= (1LL << 31))
    return fail(Q3L_EUNSUPPORTED, "B*L=%lld tokens with row stride %lld exceeds the 2 GiB "
                "offset range of the bf16 attention kernels", (long long)T,
                (long long)ld_max);
  return Q3L_OK;
}

q3l_status q3l_attention_fwd(int32_t dtype, int32_t B, int32_t L, int32_t h_q, int32_t h_kv,
                             int32_t d_h, const void* q, int64_t ldq, const void* k,
                             int64_t ldk, const void* v, int64_t ldv, void* o, int64_t ldo,
                             float* lse, void* stream) {
  q3l_status st = check_attn(dtype, B, L, h_q, h_kv, d_h);
  if (st != Q3L_OK) return st;
  Q3L_CHECK_PTR(q, "q"); Q3L_CHECK_PTR(k, "k"); Q3L_CHECK_PTR(v, "v");
  Q3L_CHECK_PTR(o, "o"); Q3L_CHECK_PTR(lse, "lse");
  if (ldq < (int64_t)h_q * d_h || ldk < (int64_t)h_kv * d_h || ldv < (int64_t)h_kv * d_h ||
      ldo < (int64_t)h_q * d_h || ldq % 8 || ldk % 8 || ldv % 8 || ldo % 8)
    return fail(Q3L_EINVAL, "row strides too small or not multiples of 8");
  if ((st = check_attn_range(dtype, B, L, h_q,
                             std::max(std::max(ldq, ldk), std::max(ldv, ldo)))) != Q3L_OK)
    return st;
  AttnArgs a{};
  a.B = B; a.L = L; a.h_q = h_q; a.h_kv = h_kv; a.d_h = d_h;
  a.q = q; a.ldq = ldq; a.k = k; a.ldk = ldk; a.v = v; a.ldv = ldv;
  a.o = o; a.ldo = ldo; a.lse = lse;
  Q3L_HIP(attn_fwd(dtype, a, static_cast<hipStream_t>(stream)));
  return Q3L_OK;
}

q3l_status q3l_attention_fwd_block(int32_t dtype, int32_t B, int32_t L, int32_t h_q,
                                   int32_t h_kv, int32_t d_h, const void* q, int64_t ldq,
                                   const void* k, int64_t ldk, const void* v, int64_t ldv,
                                   int32_t k0, int32_t k1, float* m, float* l, float* acc,
                                   void* stream) {
  q3l_status st = check_attn(dtype, B, L, h_q, h_kv, d_h);
  if (st != Q3L_OK) return st;
  if (k0 < 0 || k1 <= k0 || k1 > L)
    return fail(Q3L_EINVAL, "key range [%d, %d) must satisfy 0 <= k0 < k1 <= L=%d", k0, k1, L);
  Q3L_CHECK_PTR(q, "q"); Q3L_CHECK_PTR(k, "k"); Q3L_CHECK_PTR(v, "v");
  Q3L_CHECK_PTR(m, "m"); Q3L_CHECK_PTR(l, "l"); Q3L_CHECK_PTR(acc, "acc");
  if (ldq < (int64_t)h_q * d_h || ldk < (int64_t)h_kv * d_h || ldv < (int64_t)h_kv * d_h ||
      ldq % 8 || ldk % 8 || ldv % 8)
    return fail(Q3L_EINVAL, "row strides too small or not multiples of 8");
  if ((st = check_attn_range(dtype, B, L, h_q, std::max(std::max(ldq, ldk), ldv))) != Q3L_OK)
    return st;
  AttnArgs a{};
  a.B = B; a.L = L; a.h_q = h_q; a.h_kv = h_kv; a.d_h = d_h;
  a.q = q; a.ldq = ldq; a.k = k; a.ldk = ldk; a.v = v; a.ldv = ldv;
  a.k_lo = k0; a.k_hi = k1;
  a.m_out = m; a.l_out = l; a.acc = acc; a.ld_acc = (int64_t)h_q * d_h;
  Q3L_HIP(attn_block(dtype, a, static_cast<hipStream_t>(stream)));
  return Q3L_OK;
}

q3l_status q3l_attention_merge(int32_t B, int32_t L, int32_t h_q, int32_t d_h, float* m,
                               float* l, float* acc, const float* m2, const float* l2,
                               const float* acc2, void* stream) {
  if (B <= 0 || L <= 0 || h_q <= 0) return fail(Q3L_EINVAL, "need positive B, L, h_q");
  if (d_h != 64 && d_h != 128) return fail(Q3L_EUNSUPPORTED, "d_h must be 64 or 128");
  Q3L_CHECK_PTR(m, "m"); Q3L_CHECK_PTR(l, "l"); Q3L_CHECK_PTR(acc, "acc");
  Q3L_CHECK_PTR(m2, "m2"); Q3L_CHECK_PTR(l2, "l2"); Q3L_CHECK_PTR(acc2, "acc2");
  Q3L_HIP(attn_state_merge(B, L, h_q, d_h, m, l, acc, m2, l2, acc2,
                           static_cast<hipStream_t>(stream)));
  return Q3L_OK;
}

q3l_status q3l_attention_finish(int32_t dtype, int32_t B, int32_t L, int32_t h_q, int32_t d_h,
                                const float* m, const float* l, const float* acc, void* o,
                                int64_t ldo, float* lse, void* stream) {
  if (dtype != Q3L_F32 && dtype != Q3L_BF16) return fail(Q3L_EINVAL, "bad dtype");
  if (B <= 0 || L <= 0 || h_q <= 0) return fail(Q3L_EINVAL, "need positive B, L, h_q");
  if (d_h != 64 && d_h != 128) return fail(Q3L_EUNSUPPORTED, "d_h must be 64 or 128");
  if (ldo < (int64_t)h_q * d_h || ldo % 8) return fail(Q3L_EINVAL, "bad ldo");
  Q3L_CHECK_PTR(m, "m"); Q3L_CHECK_PTR(l, "l"); Q3L_CHECK_PTR(acc, "acc");
  Q3L_CHECK_PTR(o, "o"); Q3L_CHECK_PTR(lse, "lse");
  Q3L_HIP(attn_state_finish(dtype, B, L, h_q, d_h, m, l, acc, o, ldo, lse,
                            static_cast<hipStream_t>(stream)));
  return Q3L_OK;
}

size_t q3l_attention_bwd_workspace_bytes(int32_t B, int32_t L, int32_t h_q) {
  if (B <= 0 || L <= 0 || h_q <= 0) return 0;
  return up((size_t)B * h_q * L * 4);
}

size_t q3l_attention_bwd_stored_ds_workspace_bytes(int32_t B, int32_t L, int32_t h_q) {
  if (B <= 0 || L <= 0 || h_q <= 0) return 0;
  return q3l_attention_bwd_workspace_bytes(B, L, h_q) + up(attn_ds_bytes(B, L, h_q));
}

q3l_status q3l_attention_bwd(int32_t dtype, int32_t B, int32_t L, int32_t h_q, int32_t h_kv,
                             int32_t d_h, const void* q, int64_t ldq, const void* k,
                             int64_t ldk, const void* v, int64_t ldv, const void* o,
                             int64_t ldo, const void* dout, int64_t lddo, const float* lse,
                             void* dq, void* dk, void* dv, void* workspace,
                             size_t workspace_bytes, void* stream) {
  q3l_status st = check_attn(dtype, B, L, h_q, h_kv, d_h);
  if (st != Q3L_OK) return st;
  Q3L_CHECK_PTR(q, "q"); Q3L_CHECK_PTR(k, "k"); Q3L_CHECK_PTR(v, "v");
  Q3L_CHECK_PTR(o, "o"); Q3L_CHECK_PTR(dout, "dout"); Q3L_CHECK_PTR(lse, "lse");
  Q3L_CHECK_PTR(dq, "dq"); Q3L_CHECK_PTR(dk, "dk"); Q3L_CHECK_PTR(dv, "dv");
  Q3L_CHECK_PTR(workspace, "workspace");
  if (workspace_bytes < q3l_attention_bwd_workspace_bytes(B, L, h_q))
    return fail(Q3L_EINVAL, "workspace too small");
  if (ldq < (int64_t)h_q * d_h || ldk < (int64_t)h_kv * d_h || ldv < (int64_t)h_kv * d_h ||
      ldo < (int64_t)h_q * d_h || lddo < (int64_t)h_q * d_h || ldq % 8 || ldk % 8 ||
      ldv % 8 || ldo % 8 || lddo % 8)
    return fail(Q3L_EINVAL, "row strides too small or not multiples of 8");
  if ((st = check_attn_range(dtype, B, L, h_q,
                             std::max(std::max(std::max(ldq, ldk), std::max(ldv, ldo)),
                                      lddo))) != Q3L_OK)
    return st;
  AttnArgs a{};
  a.B = B; a.L = L; a.h_q = h_q; a.h_kv = h_kv; a.d_h = d_h;
  a.q = q; a.ldq = ldq; a.k = k; a.ldk = ldk; a.v = v; a.ldv = ldv;
  a.o = const_cast<void*>(o); a.ldo = ldo; a.lse = const_cast<float*>(lse);
  a.dout = dout; a.lddo = lddo; a.dq = dq; a.dk = dk; a.dv = dv;
  a.delta = static_cast<float*>(workspace);
  if (dtype == Q3L_BF16 &&
      workspace_bytes >= q3l_attention_bwd_stored_ds_workspace_bytes(B, L, h_q))
    a.ds = at(workspace, q3l_attention_bwd_workspace_bytes(B, L, h_q));
  Q3L_HIP(attn_bwd(dtype, a, static_cast<hipStream_t>(stream)));
  return Q3L_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The attention backward without caller-provided scratch.  Its one scratch
// buffer (the row sums D = rowsum(dO * O), [B, h_q, L] fp32) lives in a
// file-scope device array of fixed size instead; every GPU the library runs
// on holds its own copy until the process ends.  Host code uses the array's
// device address, taken once per device with hipGetSymbolAddress (the
// array's name on the host is only a stand-in).  Nothing in it has to start
// at zero: the row-sum kernel writes every row sum the later kernels read.
// ---------------------------------------------------------------------------
namespace {
constexpr size_t kScratchFloats = size_t(1) << 22;   // 16 MiB: B*h_q*L <= 4M
__device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];

// The current device's address of `scratch` (taken on the first call on
// that device; a race between two first calls stores the same address).
q3l_status scratch_address(void** out) {
  int dev = 0;
  Q3L_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(Q3L_EUNSUPPORTED, "device %d beyond the %d this build tracks", dev,
                kMaxScratchDevices);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    Q3L_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(Q3L_EHIP, "hipGetSymbolAddress returned NULL for the scratch array");
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return Q3L_OK;
}
}  // namespace

extern "C" size_t q3l_attention_bwd_noalloc_max_rows(void) { return kScratchFloats; }

extern "C" q3l_status q3l_attention_bwd_noalloc(
    int32_t dtype, int32_t B, int32_t L, int32_t h_q, int32_t h_kv, int32_t d_h, const void* q,
    int64_t ldq, const void* k, int64_t ldk, const void* v, int64_t ldv, const void* o,
    int64_t ldo, const void* dout, int64_t lddo, const float* lse, void* dq, void* dk, void* dv,
    void* stream) {
  q3l_status st = check_attn(dtype, B, L, h_q, h_kv, d_h);
  if (st != Q3L_OK) return st;
  if ((int64_t)B * h_q * L > (int64_t)kScratchFloats)
    return fail(Q3L_EINVAL, "B*h_q*L = %lld exceeds the %zu row sums the built-in scratch "
                "holds; use q3l_attention_bwd with a workspace",
                (long long)B * h_q * L, kScratchFloats);
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != Q3L_OK) return st;
  return q3l_attention_bwd(dtype, B, L, h_q, h_kv, d_h, q, ldq, k, ldk, v, ldv, o, ldo, dout,
                           lddo, lse, dq, dk, dv, ws, kScratchFloats * sizeof(float), stream);
}

// ---------------------------------------------------------------------------
// The model around a stack of layers: embedding gather, the layers, the final
// RMSNorm and the tied output projection, and the backward in reverse.
// ---------------------------------------------------------------------------
namespace {

constexpr int64_t kModelMaxTokens = 262144;   // the embedding scatter's link scan

struct ModelSaved {
  size_t xs;        // (n_layers + 1) layer inputs / the last output, [T, d] each
  size_t x_stride;  // bytes between them
  size_t hf, rf;    // final norm output [T, d] and its rstd [T] fp32
  size_t layers;    // n_layers layer saved blocks (no recompute)
  size_t layer_stride;
  size_t total;
};

ModelSaved model_saved_layout(const q3l_model_cfg& c) {
  const Dims m = dims_of(c.layer);
  ModelSaved s{};
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += up(bytes); return o; };
  s.x_stride = up(m.T * m.d * m.es);
  s.xs = take(s.x_stride * (size_t)(c.n_layers + 1));
  s.hf = take(m.T * m.d * m.es);
  s.rf = take(m.T * 4);
  s.layer_stride = up(saved_layout(c.layer).total);
  s.layers = take(c.recompute ? 0 : s.layer_stride * (size_t)c.n_layers);
  s.total = off;
  return s;
}

// Forward scratch: two x buffers and hf / rf (inference), and one layer's
// forward workspace.
struct ModelFwdWs { size_t xa, xb, hf, rf, layer, layer_bytes, total; };
ModelFwdWs model_fwd_ws(const q3l_model_cfg& c) {
  const Dims m = dims_of(c.layer);
  ModelFwdWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += up(bytes); return o; };
  w.xa = take(m.T * m.d * m.es);
  w.xb = take(m.T * m.d * m.es);
  w.hf = take(m.T * m.d * m.es);
  w.rf = take(m.T * 4);
  w.layer_bytes = saved_layout(c.layer).wt;
  w.layer = take(w.layer_bytes);
  w.total = off;
  return w;
}

// Backward scratch: the layer backward's workspace, two dx buffers, dhf, the
// final norm's partial sums, the embedding scatter's links, a layer's saved
// block and output for recomputation, and (bf16) the transposed operands of
// the output projection's two GEMMs.
struct ModelBwdWs {
  size_t layer, layer_bytes, dxa, dxb, dhf, wpart, next, first, rsaved, ry, et, dlt, hft, total;
};
ModelBwdWs model_bwd_ws(const q3l_model_cfg& c) {
  const Dims m = dims_of(c.layer);
  ModelBwdWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += up(bytes); return o; };
  w.layer_bytes = bwd_layout(c.layer).total;
  w.layer = take(w.layer_bytes);
  w.dxa = take(m.T * m.d * m.es);
  w.dxb = take(m.T * m.d * m.es);
  w.dhf = take(m.T * m.d * m.es);
  w.wpart = take((size_t)rmsnorm_bwd_max_parts() * m.d * 4);
  w.next = take(m.T * 4);
  w.first = take(m.T * 4);
  w.rsaved = take(c.recompute ? saved_layout(c.layer).total : 0);
  w.ry = take(c.recompute ? m.T * m.d * m.es : 0);
  const size_t V = (size_t)c.vocab, Tp = (size_t)pad8(m.T);
  const bool bt = c.layer.dtype == Q3L_BF16;
  w.et = take(bt ? (size_t)m.d * V * 2 : 0);
  w.dlt = take(bt ? V * Tp * 2 : 0);
  w.hft = take(bt ? (size_t)m.d * Tp * 2 : 0);
  w.total = off;
  return w;
}

q3l_status model_validate(const q3l_model_cfg* c) {
  if (!c) return fail(Q3L_EINVAL, "model cfg is NULL");
  q3l_status st = validate(&c->layer);
  if (st != Q3L_OK) return st;
  if (c->layer.tp_partial) return fail(Q3L_EUNSUPPORTED, "a model stack has no tp_partial layers");
  if (c->n_layers < 0) return fail(Q3L_EINVAL, "n_layers=%d is negative", c->n_layers);
  if (c->vocab <= 0 || c->vocab % 8) return fail(Q3L_EINVAL, "vocab=%d must be a positive multiple of 8", c->vocab);
  if (c->recompute != 0 && c->recompute != 1) return fail(Q3L_EINVAL, "recompute must be 0 or 1");
  const int64_t T = (int64_t)c->layer.B * c->layer.L, V = c->vocab, d = c->layer.d;
  if (T > kModelMaxTokens)
    return fail(Q3L_EUNSUPPORTED, "B*L=%lld exceeds the %lld tokens of the embedding scatter",
                (long long)T, (long long)kModelMaxTokens);
  if (c->layer.dtype == Q3L_BF16 &&
      ((T + 8) * V * 2 >= (1LL << 31) || (V + 8) * d * 2 >= (1LL << 31) ||
       (V + 8) * pad8(T) * 2 >= (1LL << 31)))
    return fail(Q3L_EUNSUPPORTED, "logits [%lld, %lld] or the table exceed the 2 GiB offset "
                "range of the bf16 GEMM", (long long)T, (long long)V);
  return Q3L_OK;
}

q3l_status check_model_weights(const q3l_model_cfg& c, const q3l_model_weights* w) {
  if (!w) return fail(Q3L_EINVAL, "model weights struct is NULL");
  Q3L_CHECK_PTR(w->embed, "w.embed");
  Q3L_CHECK_PTR(w->final_norm, "w.final_norm");
  if (c.n_layers > 0 && !w->layers) return fail(Q3L_EINVAL, "w.layers is NULL");
  for (int i = 0; i < c.n_layers; ++i) {
    const q3l_status st = check_weights(&w->layers[i], c.layer.qk_norm != 0);
    if (st != Q3L_OK) {
      const std::string msg = g_err;
      return fail(st, "layer %d: %s", i, msg.c_str());
    }
  }
  return Q3L_OK;
}

}  // namespace

extern "C" {

q3l_status q3l_model_validate(const q3l_model_cfg* cfg) {
  const q3l_status st = model_validate(cfg);
  if (st == Q3L_OK) g_err.clear();
  return st;
}

size_t q3l_model_saved_bytes(const q3l_model_cfg* cfg) {
  if (model_validate(cfg) != Q3L_OK) return 0;
  return model_saved_layout(*cfg).total;
}

size_t q3l_model_workspace_bytes(const q3l_model_cfg* cfg, int backward) {
  if (model_validate(cfg) != Q3L_OK) return 0;
  return backward ? model_bwd_ws(*cfg).total : model_fwd_ws(*cfg).total;
}

q3l_status q3l_model_forward(const q3l_model_cfg* cfg, const q3l_model_weights* w,
                             const int32_t* ids, void* logits, void* saved, void* workspace,
                             size_t workspace_bytes, void* stream, const q3l_exec* exec) {
  q3l_status st = model_validate(cfg);
  if (st != Q3L_OK) return st;
  const q3l_model_cfg& c = *cfg;
  if ((st = check_model_weights(c, w)) != Q3L_OK) return st;
  Q3L_CHECK_PTR(ids, "ids");
  Q3L_CHECK_PTR(logits, "logits");
  Q3L_CHECK_PTR(workspace, "workspace");
  if (saved) Q3L_CHECK_PTR(saved, "saved");
  if (exec && (exec->marks || exec->n_marks))
    return fail(Q3L_EINVAL, "exec.marks are per layer call; pass none to the model calls");
  if (exec && exec->side_stream && (!exec->fork_event || !exec->join_event))
    return fail(Q3L_EINVAL, "exec.side_stream needs exec.fork_event and exec.join_event");
  const ModelFwdWs FW = model_fwd_ws(c);
  if (workspace_bytes < FW.total)
    return fail(Q3L_EINVAL, "workspace holds %zu bytes, %zu needed", workspace_bytes, FW.total);
  const ModelSaved MS = model_saved_layout(c);
  const Dims m = dims_of(c.layer);
  const int dt = c.layer.dtype;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Layer inputs: in `saved` for a training forward, else two alternating
  // scratch buffers.
  auto xbuf = [&](int i) -> char* {
    if (saved) return at(saved, MS.xs + MS.x_stride * (size_t)i);
    return at(workspace, (i & 1) ? FW.xb : FW.xa);
  };
  char* hf = saved ? at(saved, MS.hf) : at(workspace, FW.hf);
  float* rf = reinterpret_cast<float*>(saved ? at(saved, MS.rf) : at(workspace, FW.rf));
  Q3L_HIP(embed_gather(dt, m.T, m.d, c.vocab, ids, w->embed, xbuf(0), s));
  for (int i = 0; i < c.n_layers; ++i) {
    q3l_outputs out{};
    out.y = xbuf(i + 1);
    void* ls = (saved && !c.recompute) ? at(saved, MS.layers + MS.layer_stride * (size_t)i)
                                       : nullptr;
    st = q3l_layer_forward(&c.layer, &w->layers[i], xbuf(i), &out, ls,
                           at(workspace, FW.layer), FW.layer_bytes, stream, exec);
    if (st != Q3L_OK) return st;
  }
  Q3L_HIP(rmsnorm_fwd(dt, m.T, m.d, xbuf(c.n_layers), w->final_norm, c.layer.eps, hf, rf, s));
  // Output projection, tied to the embedding table: logits = hf E^T.
  GemmArgs g{};
  g.a = kop(hf, m.d, (int)m.T);
  g.b = kop(w->embed, m.d, c.vocab);
  g.M = (int)m.T; g.N = c.vocab; g.K = m.d;
  g.epi = epi_store(logits, c.vocab, nullptr, 0);
  Q3L_HIP(gemm(dt, g, s));
  g_err.clear();
  return Q3L_OK;
}

q3l_status q3l_model_backward(const q3l_model_cfg* cfg, const q3l_model_weights* w,
                              const int32_t* ids, const void* dlogits, const void* saved,
                              const q3l_model_grads* grads, int flags, void* workspace,
                              size_t workspace_bytes, void* stream) {
  q3l_status st = model_validate(cfg);
  if (st != Q3L_OK) return st;
  const q3l_model_cfg& c = *cfg;
  if ((st = check_model_weights(c, w)) != Q3L_OK) return st;
  if (flags & ~Q3L_BWD_ACCUMULATE)
    return fail(Q3L_EINVAL, "model backward flags: only Q3L_BWD_ACCUMULATE (0x%x given)", flags);
  const int acc = (flags & Q3L_BWD_ACCUMULATE) ? 1 : 0;
  Q3L_CHECK_PTR(ids, "ids");
  Q3L_CHECK_PTR(dlogits, "dlogits");
  Q3L_CHECK_PTR(saved, "saved");
  Q3L_CHECK_PTR(workspace, "workspace");
  if (!grads) return fail(Q3L_EINVAL, "grads struct is NULL");
  Q3L_CHECK_PTR(grads->embed, "grads.embed");
  Q3L_CHECK_PTR(grads->final_norm, "grads.final_norm");
  if (c.n_layers > 0 && !grads->layers) return fail(Q3L_EINVAL, "grads.layers is NULL");
  const ModelBwdWs BW = model_bwd_ws(c);
  if (workspace_bytes < BW.total)
    return fail(Q3L_EINVAL, "workspace holds %zu bytes, %zu needed", workspace_bytes, BW.total);
  const ModelSaved MS = model_saved_layout(c);
  const Dims m = dims_of(c.layer);
  const int dt = c.layer.dtype;
  const bool bt = dt == Q3L_BF16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int T = (int)m.T, Tp = (int)pad8(m.T), V = c.vocab, d = m.d;
  auto xin = [&](int i) { return at(saved, MS.xs + MS.x_stride * (size_t)i); };
  const char* hf = at(saved, MS.hf);
  const float* rf = reinterpret_cast<const float*>(at(saved, MS.rf));
  char* dhf = at(workspace, BW.dhf);
  // Output projection: dhf = dlogits E, dE (+)= dlogits^T hf.
  {
    GemmArgs g{};
    g.a = kop(dlogits, V, T);
    if (bt) {
      char* et = at(workspace, BW.et);
      const TransposeJob job{w->embed, d, et, V, V, V, d};
      Q3L_HIP(transpose_bf16_batch(&job, 1, s));
      g.b = kop(et, V, d);
    } else {
      g.b = rop(w->embed, d, d);
    }
    g.M = T; g.N = d; g.K = V;
    g.epi = epi_store(dhf, d, nullptr, 0);
    Q3L_HIP(gemm(dt, g, s));
  }
  {
    GemmArgs g{};
    if (bt) {
      char* dlt = at(workspace, BW.dlt);
      char* hft = at(workspace, BW.hft);
      const TransposeJob jobs[2] = {{dlogits, V, dlt, Tp, T, Tp, V}, {hf, d, hft, Tp, T, Tp, d}};
      Q3L_HIP(transpose_bf16_batch(jobs, 2, s));
      g.a = kop(dlt, Tp, V);
      g.b = kop(hft, Tp, d);
      g.K = Tp;
    } else {
      g.a = rop(dlogits, V, V);
      g.b = rop(hf, d, d);
      g.K = T;
    }
    g.M = V; g.N = d;
    g.epi = epi_wgrad(grads->embed, d, acc);
    Q3L_HIP(gemm(dt, g, s));
  }
  // Final RMSNorm.
  char* dxs[2] = {at(workspace, BW.dxa), at(workspace, BW.dxb)};
  {
    float* wp = reinterpret_cast<float*>(at(workspace, BW.wpart));
    int np = 0;
    Q3L_HIP(rmsnorm_bwd(dt, m.T, d, dhf, xin(c.n_layers), rf, w->final_norm, nullptr, dxs[0],
                        wp, &np, s));
    Q3L_HIP(reduce_rows(wp, np, d, grads->final_norm, acc, s));
  }
  // Layers, last first.
  int cur = 0;
  for (int i = c.n_layers - 1; i >= 0; --i) {
    const void* ls;
    if (c.recompute) {
      q3l_outputs out{};
      out.y = at(workspace, BW.ry);
      void* rs = at(workspace, BW.rsaved);
      st = q3l_layer_forward(&c.layer, &w->layers[i], xin(i), &out, rs, nullptr, 0, stream,
                             nullptr);
      if (st != Q3L_OK) return st;
      ls = rs;
    } else {
      ls = at(saved, MS.layers + MS.layer_stride * (size_t)i);
    }
    st = q3l_layer_backward(&c.layer, &w->layers[i], xin(i), dxs[cur], ls, dxs[cur ^ 1],
                            &grads->layers[i], Q3L_BWD_INPUT | Q3L_BWD_WEIGHT | flags,
                            at(workspace, BW.layer), BW.layer_bytes, stream, nullptr);
    if (st != Q3L_OK) return st;
    cur ^= 1;
  }
  // Embedding: scatter-add dx_0 into the table's gradient (after the output
  // projection's part, so the order of the two additions is fixed).
  Q3L_HIP(embed_scatter_add(dt, T, d, V, ids, dxs[cur],
                            reinterpret_cast<int32_t*>(at(workspace, BW.next)),
                            reinterpret_cast<int32_t*>(at(workspace, BW.first)), grads->embed,
                            s));
  g_err.clear();
  return Q3L_OK;
}

}  // extern "C"
