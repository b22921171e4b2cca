// Host side of the C ABI declared in include/q3layer.h: argument validation,
// the layout of the saved tensors and of the workspace, and the launch
// sequence of the layer's forward (walkthrough page, Steps 1-10) and
// backward (the same steps' adjoints in reverse order).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
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
  // Transposed copies for the backward (bf16): the weights, then xn^T.
  s.wt = off;
  if (c.dtype == Q3L_BF16) {
    take((size_t)m.ffn * m.d * 2);
    take((size_t)m.d * 2 * m.ffn * 2);
    take((size_t)m.qd * m.d * 2);
    take((size_t)m.d * m.nqkv * 2);
  }
  s.xnt = off;
  if (c.dtype == Q3L_BF16) take((size_t)m.d * ((m.T + 7) / 8 * 8) * 2);
  s.total = off;
  return s;
}

// Offsets of the four transposed weights inside the saved wt region.
struct WtLayout { size_t down, gu, o, qkv; };
WtLayout wt_layout(const q3l_layer_cfg& c) {
  const size_t ffn = (size_t)c.d_ffn, d = (size_t)c.d;
  const size_t qd = (size_t)c.h_q * c.d_h, nqkv = qd + 2 * (size_t)c.h_kv * c.d_h;
  WtLayout w{};
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += up(bytes); return o; };
  w.down = take(ffn * d * 2);
  w.gu = take(d * 2 * ffn * 2);
  w.o = take(qd * d * 2);
  w.qkv = take(d * nqkv * 2);
  return w;
}

struct BwdWs {
  size_t dgu, dhn, dh, dO, delta, dqk, dqkv, dxn, wpart, qpart, kpart;
  // bf16 only: three scratch buffers for the transposed operands of the
  // weight-gradient GEMMs ([features, Tp]).  (The transposed weights are in
  // the saved block.)
  size_t tA, tB, tC;
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
  w.wpart = take((size_t)rmsnorm_bwd_max_parts() * m.d * 4);
  w.qpart = take((size_t)qknorm_bwd_max_parts() * m.dh * 4);
  w.kpart = take((size_t)qknorm_bwd_max_parts() * m.dh * 4);
  if (c.dtype == Q3L_BF16) {
    const size_t Tp = (size_t)pad8(m.T);
    w.tA = take((size_t)std::max<int64_t>(std::max<int64_t>(2LL * m.ffn, m.nqkv), m.d) * Tp * 2);
    w.tB = take((size_t)std::max<int64_t>(std::max<int64_t>(m.ffn, m.qd), m.d) * Tp * 2);
    w.tC = take((size_t)m.d * Tp * 2);
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

}  // namespace
}  // namespace q3l

using namespace q3l;

extern "C" {

const char* q3l_last_error(void) { return g_err.c_str(); }
int q3l_version(void) { return Q3L_VERSION; }

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

// ---- second stream ------------------------------------------------------
// One per device, created on first use and kept for the process: work that
// only depends on the call's inputs (the backward's transposed copies) runs
// on it beside the attention step, forked from and joined back into the
// caller's stream with events.  Default priority.  The mutex keeps one
// call's record / wait pairs together when several host threads share a
// device.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxDevices = 64;
std::mutex g_side_mu;
SideStream g_side[kMaxDevices];

hipError_t side_stream(SideStream** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_side_mu);
  SideStream& sd = g_side[dev];
  if (!sd.s) {
    // All three or none: a partial failure releases what was created.
    hipEvent_t f = nullptr, j = nullptr;
    hipStream_t st = nullptr;
    if ((e = hipEventCreateWithFlags(&f, hipEventDisableTiming)) == hipSuccess &&
        (e = hipEventCreateWithFlags(&j, hipEventDisableTiming)) == hipSuccess &&
        (e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking)) == hipSuccess) {
      sd.fork = f;
      sd.join = j;
      sd.s = st;
    } else {
      if (f) (void)hipEventDestroy(f);
      if (j) (void)hipEventDestroy(j);
      return e;
    }
  }
  *out = &sd;
  return hipSuccess;
}

// The copies the bf16 backward reads in K-contiguous form, from inputs the
// forward already has: the seven projection weights transposed to [in, out]
// (one launch), and xn^T [d, Tp].
hipError_t transposed_copies(const q3l_layer_cfg& c, const q3l_weights* w, const void* xn,
                             char* wt, char* xnt, hipStream_t s) {
  const Dims m = dims_of(c);
  const WtLayout o = wt_layout(c);
  const int d = m.d, ffn = m.ffn, qd = m.qd, kvd = m.kvd;
  const int T = (int)m.T, Tp = (int)((m.T + 7) / 8 * 8);
  char* wt_down = wt + o.down;
  char* wt_gu = wt + o.gu;
  char* wt_o = wt + o.o;
  char* wt_qkv = wt + o.qkv;
  const TransposeJob jobs[8] = {
      {w->down, ffn, wt_down, d, d, d, ffn},
      {w->gate, d, wt_gu, 2 * (int64_t)ffn, ffn, ffn, d},
      {w->up, d, wt_gu + (size_t)ffn * 2, 2 * (int64_t)ffn, ffn, ffn, d},
      {w->o, qd, wt_o, d, d, d, qd},
      {w->q, d, wt_qkv, m.nqkv, qd, qd, d},
      {w->k, d, wt_qkv + (size_t)qd * 2, m.nqkv, kvd, kvd, d},
      {w->v, d, wt_qkv + (size_t)(qd + kvd) * 2, m.nqkv, kvd, kvd, d},
      {xn, d, xnt, Tp, T, Tp, d}};
  return transpose_bf16_batch(jobs, 8, s);
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
                             void* workspace, size_t workspace_bytes, void* stream) {
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
  const Dims m = dims_of(c);
  const int dt = c.dtype;
  hipStream_t s = static_cast<hipStream_t>(stream);
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

  // The second stream (bf16 training forward) is obtained before anything
  // is enqueued, so a failure to create it leaves no work behind.
  SideStream* sd = nullptr;
  if (dt == Q3L_BF16 && saved) Q3L_HIP(side_stream(&sd));
  // Step 1: input RMSNorm.
  Q3L_HIP(rmsnorm_fwd(dt, m.T, m.d, x, w->in_norm, c.eps, xn, rstd1, s));
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
  // Steps 3-4: per-head q/k RMSNorm, then RoPE.
  Q3L_HIP(rope_table(m.L, m.dh, c.rope_theta, cs, sn, s));
  Q3L_HIP(qknorm_rope_fwd(dt, m.B, m.L, m.hq, m.hkv, m.dh, c.qk_norm, c.eps, qkv,
                          m.nqkv, w->q_norm, w->k_norm, cs, sn, qkr, m.nqk, rq, rk, s));
  // Step 5: causal GQA attention.
  {
    AttnArgs a{};
    a.B = m.B; a.L = m.L; a.h_q = m.hq; a.h_kv = m.hkv; a.d_h = m.dh;
    a.q = qkr; a.ldq = m.nqk;
    a.k = static_cast<const char*>(qkr) + (size_t)m.qd * m.es; a.ldk = m.nqk;
    a.v = qkvp + (size_t)(m.qd + m.kvd) * m.es; a.ldv = m.nqkv;
    a.o = ao; a.ldo = m.qd; a.lse = lse;
    if (sd) {
      // The backward's transposed copies on the second stream, beside the
      // attention kernel.  The lock keeps this call's record / wait pairs on
      // the shared events together.
      std::lock_guard<std::mutex> lk(g_side_mu);
      Q3L_HIP(hipEventRecord(sd->fork, s));
      Q3L_HIP(hipStreamWaitEvent(sd->s, sd->fork, 0));
      const hipError_t e1 = transposed_copies(c, w, xn, at(S, L.wt), at(S, L.xnt), sd->s);
      const hipError_t e2 = hipEventRecord(sd->join, sd->s);
      const hipError_t e3 = attn_fwd(dt, a, s);
      // Joined whatever happened above, so nothing of this call is left
      // running unordered with the caller's stream.
      const hipError_t e4 = hipStreamWaitEvent(s, sd->join, 0);
      Q3L_HIP(e1);
      Q3L_HIP(e2);
      Q3L_HIP(e3);
      Q3L_HIP(e4);
    } else {
      Q3L_HIP(attn_fwd(dt, a, s));
    }
  }
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
  // Step 8: post-attention RMSNorm.
  Q3L_HIP(rmsnorm_fwd(dt, m.T, m.d, h, w->post_norm, c.eps, hn, rstd2, s));
  // Step 9: gate/up as one GEMM over interleaved rows, silu(g) * u fused.
  Q3L_HIP(gemm(dt, swiglu_args(hn, m.d, (int)m.T, w->gate, w->up, m.ffn, f,
                               saved ? gu : nullptr), s));
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
  g_err.clear();
  return Q3L_OK;
}

q3l_status q3l_layer_backward(const q3l_layer_cfg* cfg, const q3l_weights* w,
                              const void* x, const void* dy, const void* saved,
                              void* dx, const q3l_grads* grads, int flags,
                              void* workspace, size_t workspace_bytes, void* stream) {
  q3l_status st = validate(cfg);
  if (st != Q3L_OK) return st;
  const q3l_layer_cfg& c = *cfg;
  if (c.tp_partial)
    return fail(Q3L_EUNSUPPORTED, "backward of a tp_partial layer is not provided");
  if ((st = check_weights(w, c.qk_norm != 0)) != Q3L_OK) return st;
  if (flags & ~(Q3L_BWD_INPUT | Q3L_BWD_WEIGHT | Q3L_BWD_ACCUMULATE))
    return fail(Q3L_EINVAL, "unknown flag bits 0x%x", flags);
  const bool want_dx = flags & Q3L_BWD_INPUT, want_w = flags & Q3L_BWD_WEIGHT;
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
  if (!want_dx && !want_w) { g_err.clear(); return Q3L_OK; }

  const q3l_saved_layout L = saved_layout(c);
  const Dims m = dims_of(c);
  const int dt = c.dtype;
  hipStream_t s = static_cast<hipStream_t>(stream);
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
  float* wpart = reinterpret_cast<float*>(at(workspace, W.wpart));
  float* qpart = reinterpret_cast<float*>(at(workspace, W.qpart));
  float* kpart = reinterpret_cast<float*>(at(workspace, W.kpart));
  const int T = (int)m.T;

  // bf16: every backward GEMM runs in the matrix-core kernel's K-contiguous
  // form.  The weights transposed to [in, out], and xn^T, come from the
  // saved block (the forward wrote them); the other operands of the
  // weight-gradient GEMMs are transposed to [features, T] (T padded to a
  // multiple of 8 with zeros) into reused scratch buffers.
  const bool bt = dt == Q3L_BF16;
  const int Tp = (int)pad8(m.T);
  const WtLayout WT = wt_layout(c);
  const char* wtb = bt ? at(saved, L.wt) : nullptr;
  const char* wt_down = bt ? wtb + WT.down : nullptr;
  const char* wt_gu = bt ? wtb + WT.gu : nullptr;
  const char* wt_o = bt ? wtb + WT.o : nullptr;
  const char* wt_qkv = bt ? wtb + WT.qkv : nullptr;
  const char* xnt = bt ? at(saved, L.xnt) : nullptr;
  char* tA = bt ? at(workspace, W.tA) : nullptr;
  char* tB = bt ? at(workspace, W.tB) : nullptr;
  char* tC = bt ? at(workspace, W.tC) : nullptr;
  // Weight gradient dW[ma, nb] (+)= sum_t A[t, ma] B[t, nb] (ma, nb are
  // feature counts; A/B activations with row strides lda/ldb).  bf16: A and
  // B are transposed into tA and tB (tA_, tB_ when given); a_done / b_done
  // say that transpose is already there.
  auto wgrad = [&](const void* A, int lda, int ma, const void* B, int ldb, int nb,
                   Epilogue e, bool a_done = false, bool b_done = false,
                   char* tA_ = nullptr, char* tB_ = nullptr) -> hipError_t {
    GemmArgs g{};
    if (bt) {
      char* ta = tA_ ? tA_ : tA;
      char* tb = tB_ ? tB_ : tB;
      TransposeJob jobs[2];
      int nj = 0;
      if (!a_done) jobs[nj++] = TransposeJob{A, lda, ta, Tp, T, Tp, ma};
      if (!b_done) jobs[nj++] = TransposeJob{B, ldb, tb, Tp, T, Tp, nb};
      const hipError_t err = transpose_bf16_batch(jobs, nj, s);   // one launch
      if (err != hipSuccess) return err;
      g.a = kop(ta, Tp, ma);
      g.b = kop(tb, Tp, nb);
      g.K = Tp;
    } else {
      g.a = rop(A, lda, ma);
      g.b = rop(B, ldb, nb);
      g.K = T;
    }
    g.M = ma; g.N = nb;
    g.epi = e;
    return gemm(dt, g, s);
  };

  // Step 9 (down_proj): df = dy W_down.  fp32: fused with the SwiGLU adjoint
  // in the GEMM epilogue.  bf16: df lands in the dg half of dgu, and a
  // separate pass turns it into dg | du, writing the transposes the two
  // weight gradients read as well: [dg du]^T and f^T (an epilogue that reads
  // g, u would hold the matrix cores idle while it waits on memory).
  {
    GemmArgs g{};
    g.a = kop(dy, m.d, T);
    g.b = bt ? kop(wt_down, m.d, m.ffn) : rop(w->down, m.ffn, m.ffn);
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
  if (bt)
    Q3L_HIP(swiglu_bwd_bf16(T, Tp, m.ffn, dgu, 2 * (int64_t)m.ffn, gu, 2 * (int64_t)m.ffn,
                            dgu, 2 * (int64_t)m.ffn, want_w ? tA : nullptr, Tp,
                            want_w ? tB : nullptr, s));
  if (want_w)  // dW_down = dy^T f  (bf16: f^T already in tB)
    Q3L_HIP(wgrad(dy, m.d, m.d, f, m.ffn, m.ffn, epi_wgrad(grads->down, m.ffn, acc),
                  /*a_done=*/false, /*b_done=*/bt, tC, nullptr));
  // Step 9 (gate/up): dhn = dg W_gate + du W_up (one GEMM over stacked K).
  {
    GemmArgs g{};
    g.a = kop(dgu, 2 * (int64_t)m.ffn, T);
    if (bt) {
      g.b = kop(wt_gu, 2 * (int64_t)m.ffn, m.d);
    } else {
      g.b = rop(w->gate, m.d, m.d);
      add_seg(g.b, w->up, m.d, m.ffn);
    }
    g.M = T; g.N = m.d; g.K = 2 * m.ffn;
    g.epi = epi_store(dhn, m.d, nullptr, 0);
    Q3L_HIP(gemm(dt, g, s));
  }
  if (want_w) {  // dW_gate | dW_up = [dg du]^T hn
    Epilogue e = epi_wgrad(grads->gate, m.d, acc);
    e.cs[1] = grads->up; e.cstart[1] = m.ffn; e.cnseg = 2;
    Q3L_HIP(wgrad(dgu, 2 * m.ffn, 2 * m.ffn, hn, m.d, m.d, e, /*a_done=*/bt));
  }
  // Steps 8 and 10: post-attention RMSNorm adjoint plus the residual dy.
  {
    int np = 0;
    Q3L_HIP(rmsnorm_bwd(dt, m.T, m.d, dhn, h, rstd2, w->post_norm, dy, dh, wpart, &np, s));
    if (want_w) Q3L_HIP(reduce_rows(wpart, np, m.d, grads->post_norm, acc, s));
  }
  // Step 6: dO = dh W_o.
  {
    GemmArgs g{};
    g.a = kop(dh, m.d, T);
    g.b = bt ? kop(wt_o, m.d, m.qd) : rop(w->o, m.qd, m.qd);
    g.M = T; g.N = m.qd; g.K = m.d;
    g.epi = epi_store(dO, m.qd, nullptr, 0);
    Q3L_HIP(gemm(dt, g, s));
  }
  if (want_w)  // dW_o = dh^T O
    Q3L_HIP(wgrad(dh, m.d, m.d, ao, m.qd, m.qd, epi_wgrad(grads->o, m.qd, acc)));
  // Step 5: attention backward (P recomputed from the log-sum-exp).
  {
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
    Q3L_HIP(attn_bwd(dt, a, s));
  }
  // Steps 4-3: RoPE adjoint and q/k RMSNorm adjoint.
  {
    int np = 0;
    Q3L_HIP(qknorm_rope_bwd(dt, m.B, m.L, m.hq, m.hkv, m.dh, c.qk_norm, dqk, m.nqk,
                            qkv, m.nqkv, w->q_norm, w->k_norm, rq, rk, cs, sn, dqkv,
                            m.nqkv, qpart, kpart, &np, s));
    if (want_w && c.qk_norm) {
      Q3L_HIP(reduce_rows2(qpart, kpart, np, m.dh, grads->q_norm, grads->k_norm, acc, s));
    }
  }
  // Step 2: dxn = [dq dk dv] [W_q; W_k; W_v].
  {
    GemmArgs g{};
    g.a = kop(dqkv, m.nqkv, T);
    if (bt) {
      g.b = kop(wt_qkv, m.nqkv, m.d);
    } else {
      g.b = rop(w->q, m.d, m.d);
      add_seg(g.b, w->k, m.d, m.qd);
      add_seg(g.b, w->v, m.d, m.qd + m.kvd);
    }
    g.M = T; g.N = m.d; g.K = m.nqkv;
    g.epi = epi_store(dxn, m.d, nullptr, 0);
    Q3L_HIP(gemm(dt, g, s));
  }
  if (want_w) {  // dW_q | dW_k | dW_v = [dq dk dv]^T xn
    Epilogue e = epi_wgrad(grads->q, m.d, acc);
    e.cs[1] = grads->k; e.cstart[1] = m.qd;
    e.cs[2] = grads->v; e.cstart[2] = m.qd + m.kvd;
    e.cnseg = 3;
    // bf16: xn^T is in the saved block (written by the forward).
    Q3L_HIP(wgrad(dqkv, m.nqkv, m.nqkv, xn, m.d, m.d, e, false, bt, nullptr,
                  const_cast<char*>(xnt)));
  }
  // Step 1: input RMSNorm adjoint plus the attention residual dh.
  {
    int np = 0;
    Q3L_HIP(rmsnorm_bwd(dt, m.T, m.d, dxn, x, rstd1, w->in_norm, dh,
                        want_dx ? dx : nullptr, wpart, &np, s));
    if (want_w) Q3L_HIP(reduce_rows(wpart, np, m.d, grads->in_norm, acc, s));
  }
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

static q3l_status check_mnk(int32_t dtype, int64_t M, int32_t N, int32_t K) {
  if (dtype != Q3L_F32 && dtype != Q3L_BF16) return fail(Q3L_EINVAL, "bad dtype");
  if (M < 0 || M > (1LL << 30) || N <= 0 || K <= 0 || N % 8 != 0 || K % 8 != 0)
    return fail(Q3L_EINVAL, "need 0 <= M <= 2^30 and N, K positive multiples of 8");
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
  GemmArgs g{};
  g.a = rop(dy, N, N);
  g.b = rop(a, K, K);
  g.M = N; g.N = K; g.K = (int)M;
  g.epi = epi_wgrad(dw, K, accumulate ? 1 : 0);
  if (M == 0) return fail(Q3L_EINVAL, "M must be positive for a weight gradient");
  Q3L_HIP(gemm(dtype, g, static_cast<hipStream_t>(stream)));
  return Q3L_OK;
}

q3l_status q3l_swiglu_fwd(int32_t dtype, int64_t M, int32_t N, int32_t K, const void* hn,
                          const void* gate, const void* up, void* f, void* gu,
                          void* stream) {
  q3l_status st = check_mnk(dtype, M, N, K);
  if (st != Q3L_OK) return st;
  Q3L_CHECK_PTR(hn, "hn"); Q3L_CHECK_PTR(gate, "gate"); Q3L_CHECK_PTR(up, "up");
  Q3L_CHECK_PTR(f, "f");
  if (gu && !aligned16(gu)) return fail(Q3L_EALIGN, "gu is not 16-byte aligned");
  Q3L_HIP(gemm(dtype, swiglu_args(hn, K, (int)M, gate, up, N, f, gu),
               static_cast<hipStream_t>(stream)));
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

size_t q3l_attention_bwd_workspace_bytes(int32_t B, int32_t L, int32_t h_q) {
  if (B <= 0 || L <= 0 || h_q <= 0) return 0;
  return up((size_t)B * h_q * L * 4);
}

q3l_status q3l_attention_bwd(int32_t dtype, int32_t B, int32_t L, int32_t h_q, int32_t h_kv,
                             int32_t d_h, const void* q, int64_t ldq, const void* k,
                             int64_t ldk, const void* v, int64_t ldv, const void* o,
                             const void* dout, int64_t ldo, const float* lse, void* dq,
                             void* dk, void* dv, void* workspace, size_t workspace_bytes,
                             void* stream) {
  q3l_status st = check_attn(dtype, B, L, h_q, h_kv, d_h);
  if (st != Q3L_OK) return st;
  Q3L_CHECK_PTR(q, "q"); Q3L_CHECK_PTR(k, "k"); Q3L_CHECK_PTR(v, "v");
  Q3L_CHECK_PTR(o, "o"); Q3L_CHECK_PTR(dout, "dout"); Q3L_CHECK_PTR(lse, "lse");
  Q3L_CHECK_PTR(dq, "dq"); Q3L_CHECK_PTR(dk, "dk"); Q3L_CHECK_PTR(dv, "dv");
  Q3L_CHECK_PTR(workspace, "workspace");
  if (workspace_bytes < q3l_attention_bwd_workspace_bytes(B, L, h_q))
    return fail(Q3L_EINVAL, "workspace too small");
  if (ldq < (int64_t)h_q * d_h || ldk < (int64_t)h_kv * d_h || ldv < (int64_t)h_kv * d_h ||
      ldo < (int64_t)h_q * d_h || ldq % 8 || ldk % 8 || ldv % 8 || ldo % 8)
    return fail(Q3L_EINVAL, "row strides too small or not multiples of 8");
  if ((st = check_attn_range(dtype, B, L, h_q,
                             std::max(std::max(ldq, ldk), std::max(ldv, ldo)))) != Q3L_OK)
    return st;
  AttnArgs a{};
  a.B = B; a.L = L; a.h_q = h_q; a.h_kv = h_kv; a.d_h = d_h;
  a.q = q; a.ldq = ldq; a.k = k; a.ldk = ldk; a.v = v; a.ldv = ldv;
  a.o = const_cast<void*>(o); a.ldo = ldo; a.lse = const_cast<float*>(lse);
  a.dout = dout; a.lddo = ldo; a.dq = dq; a.dk = dk; a.dv = dv;
  a.delta = static_cast<float*>(workspace);
  Q3L_HIP(attn_bwd(dtype, a, static_cast<hipStream_t>(stream)));
  return Q3L_OK;
}

}  // extern "C"
