// fp32 causal GQA attention for the fp32 layer (walkthrough page, Step 5):
// one wave64 per (sequence, position, head), keys visited one at a time
// with the online-softmax update.  Correctness path for small fp32 shapes;
// the bf16 path uses the matrix-core kernels.
#include "common.h"
#include "ops.h"

namespace q3l {
namespace {

struct F32P {
  int B, L, h_q, h_kv, d_h;
  const float* q; int64_t ldq;
  const float* k; int64_t ldk;
  const float* v; int64_t ldv;
  float* o; int64_t ldo;
  float* lse;
  const float* dout; int64_t lddo;
  float* dq; float* dk; float* dv;
  float* delta;
  float scale;
  int k_lo, k_hi;
  float* m_out; float* l_out; float* acc; int64_t ld_acc;
};

// d_h <= 128: each lane owns elements lane and lane + 64.
__device__ inline float wdot(const float* a, const float* b, int dh, int lane) {
  float s = 0.f;
  for (int d = lane; d < dh; d += 64) s += a[d] * b[d];
  return wave_sum(s);
}

__global__ void attn_fwd_f32_kernel(const F32P p) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= (int64_t)p.B * p.L * p.h_q) return;
  const int head = (int)(item % p.h_q);
  const int64_t tok = item / p.h_q;
  const int t = (int)(tok % p.L);
  const int64_t tok0 = tok - t;
  const int kvh = head / (p.h_q / p.h_kv);
  const float* qr = p.q + tok * p.ldq + (int64_t)head * p.d_h;
  float m = -INFINITY, l = 0.f, acc[2] = {0.f, 0.f};
  for (int s = 0; s <= t; ++s) {
    const float* kr = p.k + (tok0 + s) * p.ldk + (int64_t)kvh * p.d_h;
    const float* vr = p.v + (tok0 + s) * p.ldv + (int64_t)kvh * p.d_h;
    const float sc = wdot(qr, kr, p.d_h, lane) * p.scale;
    const float mn = fmaxf(m, sc);
    const float a = expf(m - mn), w = expf(sc - mn);
    l = l * a + w;
    for (int i = 0; i < 2; ++i) {
      const int d = lane + 64 * i;
      if (d < p.d_h) acc[i] = acc[i] * a + w * vr[d];
    }
    m = mn;
  }
  float* orow = p.o + tok * p.ldo + (int64_t)head * p.d_h;
  for (int i = 0; i < 2; ++i) {
    const int d = lane + 64 * i;
    if (d < p.d_h) orow[d] = acc[i] / l;
  }
  if (lane == 0) p.lse[((tok0 / p.L) * p.h_q + head) * p.L + t] = m + logf(l);
}

// Block state over keys [k_lo, min(k_hi, t + 1)): running maximum m (the
// exact maximum at the end), l and the unnormalised acc, (-inf, 0, 0) for a
// row with no visible key in the range.
__global__ void attn_block_f32_kernel(const F32P p) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= (int64_t)p.B * p.L * p.h_q) return;
  const int head = (int)(item % p.h_q);
  const int64_t tok = item / p.h_q;
  const int t = (int)(tok % p.L);
  const int64_t tok0 = tok - t;
  const int kvh = head / (p.h_q / p.h_kv);
  const float* qr = p.q + tok * p.ldq + (int64_t)head * p.d_h;
  float m = -INFINITY, l = 0.f, acc[2] = {0.f, 0.f};
  const int s_end = min(p.k_hi, t + 1);
  for (int s = p.k_lo; s < s_end; ++s) {
    const float* kr = p.k + (tok0 + s) * p.ldk + (int64_t)kvh * p.d_h;
    const float* vr = p.v + (tok0 + s) * p.ldv + (int64_t)kvh * p.d_h;
    const float sc = wdot(qr, kr, p.d_h, lane) * p.scale;
    const float mn = fmaxf(m, sc);
    const float a = expf(m - mn), w = expf(sc - mn);
    l = l * a + w;
    for (int i = 0; i < 2; ++i) {
      const int d = lane + 64 * i;
      if (d < p.d_h) acc[i] = acc[i] * a + w * vr[d];
    }
    m = mn;
  }
  float* arow = p.acc + tok * p.ld_acc + (int64_t)head * p.d_h;
  for (int i = 0; i < 2; ++i) {
    const int d = lane + 64 * i;
    if (d < p.d_h) arow[d] = acc[i];
  }
  if (lane == 0) {
    const int64_t si = ((tok0 / p.L) * p.h_q + head) * p.L + t;
    p.m_out[si] = m;
    p.l_out[si] = l;
  }
}

// dQ and delta = rowsum(dO * O).
__global__ void attn_dq_f32_kernel(const F32P p) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= (int64_t)p.B * p.L * p.h_q) return;
  const int head = (int)(item % p.h_q);
  const int64_t tok = item / p.h_q;
  const int t = (int)(tok % p.L);
  const int64_t tok0 = tok - t;
  const int kvh = head / (p.h_q / p.h_kv);
  const float* qr = p.q + tok * p.ldq + (int64_t)head * p.d_h;
  const float* gr = p.dout + tok * p.lddo + (int64_t)head * p.d_h;
  const float* orow = p.o + tok * p.ldo + (int64_t)head * p.d_h;
  const int64_t sidx = ((tok0 / p.L) * p.h_q + head) * p.L + t;
  const float lse = p.lse[sidx];
  const float D = wdot(gr, orow, p.d_h, lane);
  if (lane == 0) p.delta[sidx] = D;
  float acc[2] = {0.f, 0.f};
  for (int s = 0; s <= t; ++s) {
    const float* kr = p.k + (tok0 + s) * p.ldk + (int64_t)kvh * p.d_h;
    const float* vr = p.v + (tok0 + s) * p.ldv + (int64_t)kvh * p.d_h;
    const float pr = expf(wdot(qr, kr, p.d_h, lane) * p.scale - lse);
    const float ds = pr * (wdot(gr, vr, p.d_h, lane) - D);
    for (int i = 0; i < 2; ++i) {
      const int d = lane + 64 * i;
      if (d < p.d_h) acc[i] += ds * kr[d];
    }
  }
  float* dqr = p.dq + tok * p.ldq + (int64_t)head * p.d_h;
  for (int i = 0; i < 2; ++i) {
    const int d = lane + 64 * i;
    if (d < p.d_h) dqr[d] = acc[i] * p.scale;
  }
}

// dK, dV of one key of one kv head: sum over the G q heads and t >= s.
__global__ void attn_dkdv_f32_kernel(const F32P p) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= (int64_t)p.B * p.L * p.h_kv) return;
  const int kvh = (int)(item % p.h_kv);
  const int64_t tok = item / p.h_kv;
  const int s = (int)(tok % p.L);
  const int64_t tok0 = tok - s;
  const int G = p.h_q / p.h_kv;
  const float* kr = p.k + tok * p.ldk + (int64_t)kvh * p.d_h;
  const float* vr = p.v + tok * p.ldv + (int64_t)kvh * p.d_h;
  float dk[2] = {0.f, 0.f}, dv[2] = {0.f, 0.f};
  for (int j = kvh * G; j < (kvh + 1) * G; ++j) {
    for (int t = s; t < p.L; ++t) {
      const float* qr = p.q + (tok0 + t) * p.ldq + (int64_t)j * p.d_h;
      const float* gr = p.dout + (tok0 + t) * p.lddo + (int64_t)j * p.d_h;
      const int64_t sidx = ((tok0 / p.L) * p.h_q + j) * p.L + t;
      const float pr = expf(wdot(qr, kr, p.d_h, lane) * p.scale - p.lse[sidx]);
      const float ds = pr * (wdot(gr, vr, p.d_h, lane) - p.delta[sidx]);
      for (int i = 0; i < 2; ++i) {
        const int d = lane + 64 * i;
        if (d < p.d_h) {
          dv[i] += pr * gr[d];
          dk[i] += ds * qr[d];
        }
      }
    }
  }
  float* dkr = p.dk + tok * p.ldk + (int64_t)kvh * p.d_h;
  float* dvr = p.dv + tok * p.ldv + (int64_t)kvh * p.d_h;
  for (int i = 0; i < 2; ++i) {
    const int d = lane + 64 * i;
    if (d < p.d_h) {
      dkr[d] = dk[i] * p.scale;
      dvr[d] = dv[i];
    }
  }
}

F32P make_p(const AttnArgs& a) {
  F32P p{};
  p.B = a.B; p.L = a.L; p.h_q = a.h_q; p.h_kv = a.h_kv; p.d_h = a.d_h;
  p.q = (const float*)a.q; p.ldq = a.ldq;
  p.k = (const float*)a.k; p.ldk = a.ldk;
  p.v = (const float*)a.v; p.ldv = a.ldv;
  p.o = (float*)a.o; p.ldo = a.ldo;
  p.lse = a.lse;
  p.dout = (const float*)a.dout; p.lddo = a.lddo;
  p.dq = (float*)a.dq; p.dk = (float*)a.dk; p.dv = (float*)a.dv;
  p.delta = a.delta;
  p.scale = 1.0f / sqrtf((float)a.d_h);
  return p;
}

}  // namespace

hipError_t attn_fwd_bf16(const AttnArgs& a, hipStream_t s);
hipError_t attn_bwd_bf16(const AttnArgs& a, hipStream_t s);

hipError_t attn_fwd(int dtype, const AttnArgs& a, hipStream_t s) {
  if (dtype == 1) return attn_fwd_bf16(a, s);
  if (a.B <= 0 || a.L <= 0) return hipSuccess;
  const F32P p = make_p(a);
  const int64_t items = (int64_t)a.B * a.L * a.h_q;
  hipLaunchKernelGGL(attn_fwd_f32_kernel, dim3((unsigned)cdiv(items, 4)), dim3(256),
                     0, s, p);
  return hipGetLastError();
}

hipError_t attn_block_bf16(const AttnArgs& a, hipStream_t s);

hipError_t attn_block(int dtype, const AttnArgs& a, hipStream_t s) {
  if (dtype == 1) return attn_block_bf16(a, s);
  if (a.B <= 0 || a.L <= 0) return hipSuccess;
  F32P p = make_p(a);
  p.k_lo = a.k_lo; p.k_hi = a.k_hi;
  p.m_out = a.m_out; p.l_out = a.l_out; p.acc = a.acc; p.ld_acc = a.ld_acc;
  const int64_t items = (int64_t)a.B * a.L * a.h_q;
  hipLaunchKernelGGL(attn_block_f32_kernel, dim3((unsigned)cdiv(items, 4)), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t attn_bwd(int dtype, const AttnArgs& a, hipStream_t s) {
  if (dtype == 1) return attn_bwd_bf16(a, s);
  if (a.B <= 0 || a.L <= 0) return hipSuccess;
  const F32P p = make_p(a);
  const int64_t qi = (int64_t)a.B * a.L * a.h_q, ki = (int64_t)a.B * a.L * a.h_kv;
  hipLaunchKernelGGL(attn_dq_f32_kernel, dim3((unsigned)cdiv(qi, 4)), dim3(256), 0, s, p);
  hipLaunchKernelGGL(attn_dkdv_f32_kernel, dim3((unsigned)cdiv(ki, 4)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace q3l
