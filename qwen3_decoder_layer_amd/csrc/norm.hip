// Norm-family kernels of the Qwen3 decoder layer: RMSNorm forward/backward
// (walkthrough page, Steps 1 and 8), the per-head q_norm/k_norm fused with
// RoPE (Steps 3-4) and its backward, the RoPE angle table, and the column
// reduction of per-block weight-gradient partials.
//
// All of these are HBM-bound: each reads its inputs once and writes its
// outputs once with 16-byte accesses; reductions over a row stay inside a
// wave64 (shuffles), reductions over rows go through per-block partial sums.
#include <type_traits>

#include "common.h"
#include "ops.h"

namespace q3l {
namespace {

// Eight consecutive elements as fp32 (one 16-byte access for bf16, two for
// fp32).
template <class T> struct V8;
template <> struct V8<bf16_t> {
  __device__ static void load(const bf16_t* p, float f[8]) {
    const u32x4_t v = ld16(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) { f[2 * j] = lo_f(v[j]); f[2 * j + 1] = hi_f(v[j]); }
  }
  __device__ static void store(bf16_t* p, const float f[8]) {
    st16(p, u32x4_t{pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]),
                    pack2(f[6], f[7])});
  }
};
template <> struct V8<float> {
  __device__ static void load(const float* p, float f[8]) {
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(p + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) { f[j] = a[j]; f[4 + j] = b[j]; }
  }
  __device__ static void store(float* p, const float f[8]) {
    *reinterpret_cast<f32x4_t*>(p) = f32x4_t{f[0], f[1], f[2], f[3]};
    *reinterpret_cast<f32x4_t*>(p + 4) = f32x4_t{f[4], f[5], f[6], f[7]};
  }
};

// ---- RMSNorm forward: one wave per row ------------------------------------
// The row stays in registers (CPL 8-element chunks per lane, n <= 512 CPL):
// every load of the row, and of the weight, is issued before the first use,
// so each wave has the whole row in flight and x is read once.  bf16 rows
// and weights stay packed (half the registers of fp32 copies).
template <class T, int CPL>
__global__ __launch_bounds__(256) void rmsnorm_fwd_kernel(
    int64_t rows, int n, const T* __restrict__ x, const T* __restrict__ w,
    float eps, T* __restrict__ y, float* __restrict__ rstd) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const T* xr = x + row * n;
  T* yr = y + row * n;
  const int nc = n / 8;
  if constexpr (std::is_same<T, bf16_t>::value) {
    u32x4_t xv[CPL], wv[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int ch = lane + 64 * c;
      xv[c] = ch < nc ? ld16(xr + 8 * ch) : u32x4_t{0u, 0u, 0u, 0u};
      wv[c] = ch < nc ? ld16(w + 8 * ch) : u32x4_t{0u, 0u, 0u, 0u};
    }
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a = lo_f(xv[c][j]), b = hi_f(xv[c][j]);
        ss += a * a;
        ss += b * b;
      }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)n + eps);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int ch = lane + 64 * c;
      if (ch >= nc) continue;
      u32x4_t o;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        o[j] = pack2(lo_f(xv[c][j]) * r * lo_f(wv[c][j]), hi_f(xv[c][j]) * r * hi_f(wv[c][j]));
      st16(yr + 8 * ch, o);
    }
    if (lane == 0) rstd[row] = r;
  } else {
    float f[CPL][8];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int ch = lane + 64 * c;
      if (ch < nc) {
        V8<T>::load(xr + 8 * ch, f[c]);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) f[c][j] = 0.f;
      }
    }
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) ss += f[c][j] * f[c][j];
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)n + eps);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int ch = lane + 64 * c;
      if (ch >= nc) continue;
      float g[8];
      V8<T>::load(w + 8 * ch, g);
#pragma unroll
      for (int j = 0; j < 8; ++j) f[c][j] = f[c][j] * r * g[j];
      V8<T>::store(yr + 8 * ch, f[c]);
    }
    if (lane == 0) rstd[row] = r;
  }
}

// ---- RMSNorm backward -----------------------------------------------------
// Per row r (xhat = x * rstd, g = dy * w):
//   dx = rstd * (g - xhat * mean(g * xhat)) + resid
// and the block accumulates dw = sum_rows dy * xhat into one partial row.
// CPL = 8-element chunks per lane (n <= 512 * CPL).
template <class T, int CPL>
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(
    int64_t rows, int n, const T* __restrict__ dy, const T* __restrict__ x,
    const float* __restrict__ rstd, const T* __restrict__ w,
    const T* __restrict__ resid, T* __restrict__ dx, float* __restrict__ wpart) {
  extern __shared__ float sdw[];  // [n]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nc = n / 8;
  for (int i = threadIdx.x; i < n; i += 256) sdw[i] = 0.f;
  float acc[CPL][8];
#pragma unroll
  for (int c = 0; c < CPL; ++c)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[c][j] = 0.f;
  __syncthreads();

  const int64_t nwaves = (int64_t)gridDim.x * 4;
  for (int64_t row = (int64_t)blockIdx.x * 4 + wave; row < rows; row += nwaves) {
    const float r = rstd[row];
    const T* dyr = dy + row * n;
    const T* xr = x + row * n;
    float dot = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int ch = lane + 64 * c;
      if (ch < nc) {
        float a[8], b[8], ww[8];
        V8<T>::load(dyr + 8 * ch, a);
        V8<T>::load(xr + 8 * ch, b);
        V8<T>::load(w + 8 * ch, ww);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float xh = b[j] * r;
          dot += a[j] * ww[j] * xh;
          acc[c][j] += a[j] * xh;
        }
      }
    }
    dot = wave_sum(dot) / (float)n;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int ch = lane + 64 * c;
      if (ch < nc) {
        float a[8], b[8], ww[8], o[8];
        V8<T>::load(dyr + 8 * ch, a);
        V8<T>::load(xr + 8 * ch, b);
        V8<T>::load(w + 8 * ch, ww);
        float rr[8];
        if (resid) {
          V8<T>::load(resid + row * n + 8 * ch, rr);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) rr[j] = 0.f;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
          o[j] = r * (a[j] * ww[j] - b[j] * r * dot) + rr[j];
        if (dx) V8<T>::store(dx + row * n + 8 * ch, o);
      }
    }
  }
  // Waves add their partials one after another: a fixed summation order, so
  // the weight gradient is bitwise reproducible.
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int ch = lane + 64 * c;
        if (ch < nc)
#pragma unroll
          for (int j = 0; j < 8; ++j) sdw[8 * ch + j] += acc[c][j];
      }
    }
    __syncthreads();
  }
  for (int i = threadIdx.x; i < n; i += 256) wpart[(int64_t)blockIdx.x * n + i] = sdw[i];
}

// bf16 form of the same.  A workgroup (4 waves) works on one row at a time,
// each thread on CPT 8-element chunks (thread t: chunks t, t + 256, ...),
// and requests the rows it will finish next (dy, x, the residual, rstd)
// D rows ahead: while a row is reduced and written, the loads of the
// following D - 1 rows are in flight.  All accesses go through buffer
// resources, rows past the workgroup's last and chunks past the row at an
// out-of-range offset (zeros in, stores dropped), so the loop is straight-
// line code and the compiler's wait counts let the younger rows' loads stay
// in flight.  The row's dot product is summed over the 4 waves through LDS
// (one barrier per row, double-buffered by row parity); w and the weight-
// gradient sums stay in registers for the workgroup's rows, which are
// blockIdx.x, blockIdx.x + gridDim.x, ...
template <int CPT, bool RES>
__global__ __launch_bounds__(256) void rmsnorm_bwd_bf16_kernel(
    int64_t rows, int n, const bf16_t* __restrict__ dy, const bf16_t* __restrict__ x,
    const float* __restrict__ rstd, const bf16_t* __restrict__ w,
    const bf16_t* __restrict__ resid, bf16_t* __restrict__ dx, float* __restrict__ wpart) {
  constexpr int D = CPT <= 2 ? 4 : 2;   // rows in flight
  __shared__ float red[2][4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nc = n / 8;
  const int64_t G = gridDim.x, r0 = blockIdx.x;
  const int64_t nmine = r0 < rows ? (rows - 1 - r0) / G + 1 : 0;
  uint32_t coff[CPT];   // byte offset of chunk c in a row, kOOB past the row
  u32x4_t wv[CPT];
  float acc[CPT][8];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = tid + 256 * c;
    coff[c] = ch < nc ? 16u * (uint32_t)ch : kOOB;
    wv[c] = buf_ld16(buf_rsrc(w), coff[c]);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[c][j] = 0.f;
  }
  u32x4_t ra[D][CPT], rb[D][CPT], rr[RES ? D : 1][CPT];
  float rs[D];
  auto issue = [&](int64_t i, auto slot) __attribute__((always_inline)) {
    constexpr int s = decltype(slot)::value;
    const bool ok = i < nmine;
    const int64_t ro = (ok ? r0 + i * G : 0) * n;
    rs[s] = buf_ldf(buf_rsrc(rstd + (ok ? r0 + i * G : 0)), ok ? 0u : kOOB);
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const uint32_t o = ok ? coff[c] : kOOB;
      ra[s][c] = buf_ld16(buf_rsrc(dy + ro), o);
      rb[s][c] = buf_ld16(buf_rsrc(x + ro), o);
      if constexpr (RES) rr[s][c] = buf_ld16(buf_rsrc(resid + ro), o);
    }
  };
  const uint32_t dx_bytes = dx ? 0x7FFFFFFFu : 0u;   // no dx: every store dropped
  auto finish = [&](int64_t i, auto slot) __attribute__((always_inline)) {
    constexpr int s = decltype(slot)::value;
    const bool ok = i < nmine;
    const int64_t ro = (ok ? r0 + i * G : 0) * n;
    const float r = rs[s];
    float dot = 0.f;
#pragma unroll
    for (int c = 0; c < CPT; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t pa = ra[s][c][j >> 1], pb = rb[s][c][j >> 1], pw = wv[c][j >> 1];
        const float a = (j & 1) ? hi_f(pa) : lo_f(pa);
        const float xh = ((j & 1) ? hi_f(pb) : lo_f(pb)) * r;
        const float ww = (j & 1) ? hi_f(pw) : lo_f(pw);
        dot += a * ww * xh;
        acc[c][j] += a * xh;
      }
    // Unpacked copies of dy and x are not kept past the reduction, and the
    // weight-gradient sums are updated here rather than deferred (the empty
    // asm marks the registers as rewritten): fewer registers.
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      asm volatile("" : "+v"(ra[s][c]), "+v"(rb[s][c]));
#pragma unroll
      for (int j = 0; j < 8; ++j) asm volatile("" : "+v"(acc[c][j]));
    }
    dot = wave_sum(dot);
    const int par = (int)(i & 1);
    if (lane == 0) red[par][wave] = dot;
    stage_barrier();
    dot = (red[par][0] + red[par][1] + red[par][2] + red[par][3]) / (float)n;
    const __amdgpu_buffer_rsrc_t rd = buf_rsrc(dx + ro, dx_bytes);
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      float o[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t pa = ra[s][c][j >> 1], pb = rb[s][c][j >> 1], pw = wv[c][j >> 1];
        const float a = (j & 1) ? hi_f(pa) : lo_f(pa);
        const float b = (j & 1) ? hi_f(pb) : lo_f(pb);
        const float ww = (j & 1) ? hi_f(pw) : lo_f(pw);
        o[j] = r * (a * ww - b * r * dot);
        if constexpr (RES) {
          const uint32_t pr = rr[s][c][j >> 1];
          o[j] += (j & 1) ? hi_f(pr) : lo_f(pr);
        }
      }
      buf_st16(rd, ok ? coff[c] : kOOB,
               u32x4_t{pack2(o[0], o[1]), pack2(o[2], o[3]), pack2(o[4], o[5]),
                       pack2(o[6], o[7])});
    }
    issue(i + D, slot);
  };
  issue(0, std::integral_constant<int, 0>{});
  issue(1, std::integral_constant<int, 1>{});
  if constexpr (D == 4) {
    issue(2, std::integral_constant<int, 2>{});
    issue(3, std::integral_constant<int, 3>{});
  }
  for (int64_t i = 0; i < nmine; i += D) {
    finish(i, std::integral_constant<int, 0>{});
    finish(i + 1, std::integral_constant<int, 1>{});
    if constexpr (D == 4) {
      finish(i + 2, std::integral_constant<int, 2>{});
      finish(i + 3, std::integral_constant<int, 3>{});
    }
  }
  // This workgroup's weight-gradient partial row (its rows summed in order).
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = tid + 256 * c;
    if (ch < nc) {
      float* q = wpart + r0 * n + 8 * ch;
      *reinterpret_cast<f32x4_t*>(q) = f32x4_t{acc[c][0], acc[c][1], acc[c][2], acc[c][3]};
      *reinterpret_cast<f32x4_t*>(q + 4) = f32x4_t{acc[c][4], acc[c][5], acc[c][6], acc[c][7]};
    }
  }
}

constexpr int kNormBwdParts = 512;

// ---- column reduction of partial rows -------------------------------------
// A workgroup owns 64 columns; its 16 waves sum interleaved sixteenths of
// the partial rows (lanes over columns: 256-byte coalesced reads), then
// combine in a fixed order.  One launch may serve two reductions of the same
// shape (the q and k norm weights): workgroups past the first job's take
// the second.
__global__ __launch_bounds__(1024) void reduce_rows_kernel(
    const float* __restrict__ part, const float* __restrict__ part2, int nparts, int n,
    float* __restrict__ out, float* __restrict__ out2, int accumulate) {
  __shared__ float red[16][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;   // 16 waves
  const int nb = (n + 63) / 64;
  const bool second = (int)blockIdx.x >= nb;
  if (second) { part = part2; out = out2; }
  const int i = ((int)blockIdx.x - (second ? nb : 0)) * 64 + lane;
  float s = 0.f;
  if (i < n) {
#pragma unroll 8
    for (int p = wave; p < nparts; p += 16) s += part[(int64_t)p * n + i];
  }
  red[wave][lane] = s;
  __syncthreads();
  if (wave == 0 && i < n) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < 16; ++w) t += red[w][lane];
    out[i] = accumulate ? out[i] + t : t;
  }
}

// ---- RoPE angle table: angle(t, i) = t * theta^(-2i/d_h), in double --------
__global__ void rope_table_kernel(int L, int d_h, double theta,
                                  float* __restrict__ cos_t,
                                  float* __restrict__ sin_t) {
  const int half = d_h / 2;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= L * half) return;
  const int t = idx / half, i = idx % half;
  const double inv = pow(theta, -2.0 * (double)i / (double)d_h);
  const double a = (double)t * inv;
  // Reduced to [-pi, pi] first (Cody-Waite: 2 pi = C1 + C2 + C3, C1 and C2
  // with 30 significant bits, so k C1 and k C2 are exact for k < 2^22):
  // angles up to L radians would otherwise take the slow large-argument path
  // of the fp64 cos / sin; the reduced angle is exact to about 1e-16 a.
  const double C1 = 0x1.921fb54000000p+2, C2 = 0x1.10b4611800000p-28,
               C3 = 0x1.313198a2e0370p-59;
  const double k = rint(a * 0x1.45f306dc9c883p-3);   // a / (2 pi)
  const double r = ((a - k * C1) - k * C2) - k * C3;
  double sr, cr;
  sincos(r, &sr, &cr);
  cos_t[idx] = (float)cr;
  sin_t[idx] = (float)sr;
}

// Eight elements of T as the raw words of their load (bf16: four, fp32:
// eight), so a load in flight holds only its packed words.
template <class T> struct Raw8;
template <> struct Raw8<bf16_t> {
  u32x4_t w;
  __device__ void load(const bf16_t* p) { w = ld16(p); }
  __device__ void get(float f[8]) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) { f[2 * j] = lo_f(w[j]); f[2 * j + 1] = hi_f(w[j]); }
  }
};
template <> struct Raw8<float> {
  f32x4_t a, b;
  __device__ void load(const float* p) {
    a = *reinterpret_cast<const f32x4_t*>(p);
    b = *reinterpret_cast<const f32x4_t*>(p + 4);
  }
  __device__ void get(float f[8]) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) { f[j] = a[j]; f[4 + j] = b[j]; }
  }
};

// ---- q/k norm + RoPE forward ----------------------------------------------
// One wave per token.  A (token, head) vector is held by a group of LP =
// d_h/8 lanes, lane j of the group holding elements 8j..8j+7; the wave's
// 64/LP groups take HPW consecutive heads per step.  Rotate-half pairing:
// element i (< d_h/2) pairs with i + d_h/2, which sits in lane j ^ (LP/2).
// The rotation row of the token's position and the two norm weights are the
// same for every head of the token, so they are loaded once; the head
// vectors of NB steps at a time are requested together, before the first of
// them is used (NB = 5: 20 heads of 128 per request batch, the measured best
// against 10, all 40 heads of the 8B shape).
template <class T, int DH>
__global__ __launch_bounds__(256) void qknorm_rope_fwd_kernel(
    int64_t tokens, int L, int h_q, int h_kv, int qk_norm, float eps,
    const T* __restrict__ in, int64_t ld_in, const T* __restrict__ wq,
    const T* __restrict__ wk, const float* __restrict__ cos_t,
    const float* __restrict__ sin_t, T* __restrict__ out, int64_t ld_out,
    float* __restrict__ rstd_q, float* __restrict__ rstd_k) {
  constexpr int LP = DH / 8, HALF = LP / 2, HPW = 64 / LP, NB = 5;
  const int lane = threadIdx.x & 63;
  const int j = lane % LP, grp = lane / LP;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= tokens) return;
  const int heads = h_q + h_kv;
  const int pos = (int)(t % L);
  const int i0 = 8 * (j % HALF);
  const T* src = in + t * ld_in + 8 * j;
  T* dst = out + t * ld_out + 8 * j;
  for (int h0 = 0; h0 < heads; h0 += NB * HPW) {
    Raw8<T> raw[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (h0 + b * HPW >= heads) break;       // whole steps past the last head
      // Groups past the last head (final step only) read the last head again.
      raw[b].load(src + (int64_t)min(h0 + b * HPW + grp, heads - 1) * DH);
    }
    float cs[8], sn[8], wqv[8], wkv[8];
    V8<float>::load(cos_t + (int64_t)pos * (DH / 2) + i0, cs);
    V8<float>::load(sin_t + (int64_t)pos * (DH / 2) + i0, sn);
    if (qk_norm) {
      V8<T>::load(wq + 8 * j, wqv);
      V8<T>::load(wk + 8 * j, wkv);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (h0 + b * HPW >= heads) break;
      const int hh = h0 + b * HPW + grp;
      const bool isq = hh < h_q;
      float v[8];
      raw[b].get(v);
      float r = 1.f;
      if (qk_norm) {
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
        ss = group_sum(ss, LP);
        r = 1.0f / sqrtf(ss / (float)DH + eps);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = v[e] * r * (isq ? wqv[e] : wkv[e]);
      }
      float pv[8], o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = __shfl_xor(v[e], HALF, 64);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        o[e] = (j < HALF) ? v[e] * cs[e] - pv[e] * sn[e] : v[e] * cs[e] + pv[e] * sn[e];
      if (hh < heads) {
        V8<T>::store(dst + (int64_t)hh * DH, o);
        if (qk_norm && j == 0) {
          if (isq) rstd_q[t * h_q + hh] = r;
          else rstd_k[t * h_kv + (hh - h_q)] = r;
        }
      }
    }
  }
}

// ---- q/k norm + RoPE backward ---------------------------------------------
// g: gradient w.r.t. the rotated, normalised q/k.  Inverse rotation, then the
// RMSNorm adjoint per head.  Lane roles and loads as in the forward; wave w
// of the grid takes tokens w, w + (number of waves), ...  The
// weight-gradient sums dn * x_hat stay in registers (every lane with the
// same j holds the same eight weights), are added across the wave's lane
// groups, then across its four waves through LDS in a fixed order: one
// partial row of dw_q and of dw_k per workgroup.
template <class T, int DH>
__global__ __launch_bounds__(256) void qknorm_rope_bwd_kernel(
    int64_t tokens, int L, int h_q, int h_kv, int qk_norm,
    const T* __restrict__ g, int64_t ld_g, const T* __restrict__ pre,
    int64_t ld_pre, const T* __restrict__ wq, const T* __restrict__ wk,
    const float* __restrict__ rstd_q, const float* __restrict__ rstd_k,
    const float* __restrict__ cos_t, const float* __restrict__ sin_t,
    T* __restrict__ out, int64_t ld_out, float* __restrict__ wq_part,
    float* __restrict__ wk_part) {
  constexpr int LP = DH / 8, HALF = LP / 2, HPW = 64 / LP, NB = 3;
  __shared__ float sq[DH], sk[DH];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane % LP, grp = lane / LP;
  const int heads = h_q + h_kv;
  for (int i = threadIdx.x; i < DH; i += 256) { sq[i] = 0.f; sk[i] = 0.f; }
  float aq[8], ak[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) { aq[e] = 0.f; ak[e] = 0.f; }
  const int i0 = 8 * (j % HALF);
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  for (int64_t t = (int64_t)blockIdx.x * 4 + wave; t < tokens; t += nwaves) {
    const int pos = (int)(t % L);
    const T* gsrc = g + t * ld_g + 8 * j;
    const T* psrc = pre + t * ld_pre + 8 * j;
    T* dst = out + t * ld_out + 8 * j;
    for (int h0 = 0; h0 < heads; h0 += NB * HPW) {
      // Every load of the token's steps (gradients, pre-norm vectors, their
      // rstd, the rotation row, the norm weights) is issued before the
      // first use.
      Raw8<T> gr[NB], xr[NB];
      float rr[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if (h0 + b * HPW >= heads) break;
        const int hh = min(h0 + b * HPW + grp, heads - 1);
        gr[b].load(gsrc + (int64_t)hh * DH);
        rr[b] = 1.f;
        if (qk_norm) {
          xr[b].load(psrc + (int64_t)hh * DH);
          rr[b] = hh < h_q ? rstd_q[t * h_q + hh] : rstd_k[t * h_kv + (hh - h_q)];
        }
      }
      float cs[8], sn[8], wqv[8], wkv[8];
      V8<float>::load(cos_t + (int64_t)pos * (DH / 2) + i0, cs);
      V8<float>::load(sin_t + (int64_t)pos * (DH / 2) + i0, sn);
      if (qk_norm) {
        V8<T>::load(wq + 8 * j, wqv);
        V8<T>::load(wk + 8 * j, wkv);
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if (h0 + b * HPW >= heads) break;
        const int hh = h0 + b * HPW + grp;
        const bool isq = hh < h_q, ok = hh < heads;
        const float r = rr[b];
        float gv[8], pg[8], dn[8], o[8];
        gr[b].get(gv);
#pragma unroll
        for (int e = 0; e < 8; ++e) pg[e] = __shfl_xor(gv[e], HALF, 64);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          dn[e] = (j < HALF) ? gv[e] * cs[e] + pg[e] * sn[e] : gv[e] * cs[e] - pg[e] * sn[e];
        if (qk_norm) {
          float wv[8], xv[8];
          xr[b].get(xv);
#pragma unroll
          for (int e = 0; e < 8; ++e) wv[e] = isq ? wqv[e] : wkv[e];
          float dot = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) dot += dn[e] * wv[e] * xv[e] * r;
          dot = group_sum(dot, LP) / (float)DH;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float xh = xv[e] * r;
            o[e] = r * (dn[e] * wv[e] - xh * dot);
            if (ok) {
              if (isq) aq[e] += dn[e] * xh;
              else ak[e] += dn[e] * xh;
            }
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = dn[e];
        }
        if (ok) V8<T>::store(dst + (int64_t)hh * DH, o);
      }
    }
  }
  if (!qk_norm) return;
  // Lanes with the same j hold partials of the same 8 weights.
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    for (int o2 = LP; o2 < 64; o2 <<= 1) {
      aq[e] += __shfl_xor(aq[e], o2, 64);
      ak[e] += __shfl_xor(ak[e], o2, 64);
    }
  }
  __syncthreads();   // sq, sk cleared
  for (int w = 0; w < 4; ++w) {   // fixed order across waves
    if (wave == w && lane < LP) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sq[8 * j + e] += aq[e];
        sk[8 * j + e] += ak[e];
      }
    }
    __syncthreads();
  }
  for (int i = threadIdx.x; i < DH; i += 256) {
    wq_part[(int64_t)blockIdx.x * DH + i] = sq[i];
    wk_part[(int64_t)blockIdx.x * DH + i] = sk[i];
  }
}

// At most one round of workgroups: 256 CUs x 3 (the kernel's occupancy at
// d_h = 128), each wave taking several tokens (15% faster than 2048
// workgroups of one token per wave, whose ragged third round and per-
// workgroup partial sums cost more than the longer loop).
constexpr int kQkBwdParts = 768;

// Workgroups (= partial rows of the weight gradient) of the RMSNorm
// backward: bf16 at least 8 rows per workgroup, so the loads of the next rows
// overlap; fp32 at least 4 rows per wave.
int64_t rmsnorm_bwd_grid(int dtype, int64_t rows) {
  int64_t grid = dtype == 1 ? cdiv(rows, 8) : cdiv(rows, 4 * 4);
  if (grid > kNormBwdParts) grid = kNormBwdParts;
  if (grid < 1) grid = 1;
  return grid;
}

template <class T>
hipError_t rmsnorm_bwd_t(int64_t rows, int n, const void* dy, const void* x,
                         const float* rstd, const void* w, const void* resid, void* dx,
                         float* wpart, int* nparts, hipStream_t s) {
  if constexpr (std::is_same<T, bf16_t>::value) {
    const int64_t grid = rmsnorm_bwd_grid(1, rows);
    *nparts = (int)grid;
    const int cpt = (int)cdiv(n, 8 * 256);
#define Q3L_RB16K(C, R)                                                              \
  hipLaunchKernelGGL((rmsnorm_bwd_bf16_kernel<C, R>), dim3(grid), dim3(256), 0, s,   \
                     rows, n, (const bf16_t*)dy, (const bf16_t*)x, rstd,             \
                     (const bf16_t*)w, (const bf16_t*)resid, (bf16_t*)dx, wpart)
#define Q3L_RB16(C)                \
  if (resid) Q3L_RB16K(C, true);   \
  else Q3L_RB16K(C, false);
    if (cpt <= 1) { Q3L_RB16(1) }
    else if (cpt <= 2) { Q3L_RB16(2) }
    else if (cpt <= 4) { Q3L_RB16(4) }
    else return hipErrorInvalidValue;
#undef Q3L_RB16
#undef Q3L_RB16K
    return hipGetLastError();
  }
  const int cpl = (int)cdiv(n, 512);
  const int64_t grid = rmsnorm_bwd_grid(0, rows);
  *nparts = (int)grid;
  const size_t shm = (size_t)n * sizeof(float);
#define Q3L_RB(C)                                                              \
  hipLaunchKernelGGL((rmsnorm_bwd_kernel<T, C>), dim3(grid), dim3(256), shm, s, \
                     rows, n, (const T*)dy, (const T*)x, rstd, (const T*)w,    \
                     (const T*)resid, (T*)dx, wpart)
  if (cpl <= 1) Q3L_RB(1);
  else if (cpl <= 2) Q3L_RB(2);
  else if (cpl <= 4) Q3L_RB(4);
  else if (cpl <= 8) Q3L_RB(8);
  else if (cpl <= 16) Q3L_RB(16);
  else return hipErrorInvalidValue;
#undef Q3L_RB
  return hipGetLastError();
}

// Workgroups (= partial rows) of the q/k norm backward: four waves of one
// token at a time; one token per wave up to kQkBwdParts workgroups.
int64_t qknorm_bwd_grid(int64_t tokens, int heads, int d_h) {
  (void)heads; (void)d_h;
  int64_t grid = cdiv(tokens, 4);
  if (grid > kQkBwdParts) grid = kQkBwdParts;
  if (grid < 1) grid = 1;
  return grid;
}

}  // namespace

int rmsnorm_bwd_max_parts() { return kNormBwdParts; }
int qknorm_bwd_max_parts() { return kQkBwdParts; }
int rmsnorm_bwd_parts(int dtype, int64_t rows, int n) {
  (void)n;
  return (int)rmsnorm_bwd_grid(dtype, rows);
}
int qknorm_bwd_parts(int64_t tokens, int heads, int d_h) {
  return (int)qknorm_bwd_grid(tokens, heads, d_h);
}

hipError_t rmsnorm_fwd(int dtype, int64_t rows, int n, const void* x,
                       const void* w, float eps, void* y, float* rstd,
                       hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  dim3 grid((unsigned)cdiv(rows, 4)), block(256);
  const int cpl = (int)cdiv(n, 512);
#define Q3L_RF(T, C)                                                                \
  hipLaunchKernelGGL((rmsnorm_fwd_kernel<T, C>), grid, block, 0, s, rows, n,         \
                     (const T*)x, (const T*)w, eps, (T*)y, rstd)
#define Q3L_RF_ALL(T)                        \
  if (cpl <= 1) Q3L_RF(T, 1);                \
  else if (cpl <= 2) Q3L_RF(T, 2);           \
  else if (cpl <= 4) Q3L_RF(T, 4);           \
  else if (cpl <= 8) Q3L_RF(T, 8);           \
  else if (cpl <= 16) Q3L_RF(T, 16);         \
  else return hipErrorInvalidValue;
  if (dtype == 1) {
    Q3L_RF_ALL(bf16_t)
  } else {
    Q3L_RF_ALL(float)
  }
#undef Q3L_RF_ALL
#undef Q3L_RF
  return hipGetLastError();
}

hipError_t rmsnorm_bwd(int dtype, int64_t rows, int n, const void* dy,
                       const void* x, const float* rstd, const void* w,
                       const void* resid, void* dx, float* wpart, int* nparts,
                       hipStream_t s) {
  if (dtype == 1)
    return rmsnorm_bwd_t<bf16_t>(rows, n, dy, x, rstd, w, resid, dx, wpart, nparts, s);
  return rmsnorm_bwd_t<float>(rows, n, dy, x, rstd, w, resid, dx, wpart, nparts, s);
}

hipError_t reduce_rows(const float* part, int nparts, int n, float* out,
                       int accumulate, hipStream_t s) {
  hipLaunchKernelGGL(reduce_rows_kernel, dim3((unsigned)cdiv(n, 64)), dim3(1024),
                     0, s, part, nullptr, nparts, n, out, nullptr, accumulate);
  return hipGetLastError();
}

hipError_t reduce_rows2(const float* part, const float* part2, int nparts, int n,
                        float* out, float* out2, int accumulate, hipStream_t s) {
  hipLaunchKernelGGL(reduce_rows_kernel, dim3((unsigned)(2 * cdiv(n, 64))), dim3(1024),
                     0, s, part, part2, nparts, n, out, out2, accumulate);
  return hipGetLastError();
}

hipError_t rope_table(int L, int d_h, float theta, float* cos_t, float* sin_t,
                      hipStream_t s) {
  const int n = L * (d_h / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256),
                     0, s, L, d_h, (double)theta, cos_t, sin_t);
  return hipGetLastError();
}

hipError_t qknorm_rope_fwd(int dtype, int B, int L, int h_q, int h_kv,
                           int d_h, int qk_norm, float eps, const void* in,
                           int64_t ld_in, const void* wq, const void* wk,
                           const float* cos_t, const float* sin_t, void* out,
                           int64_t ld_out, float* rstd_q, float* rstd_k,
                           hipStream_t s) {
  const int64_t tokens = (int64_t)B * L;
  dim3 grid((unsigned)cdiv(tokens, 4)), block(256);   // one wave per token
#define Q3L_QF(T, D)                                                          \
  hipLaunchKernelGGL((qknorm_rope_fwd_kernel<T, D>), grid, block, 0, s,       \
                     tokens, L, h_q, h_kv, qk_norm, eps, (const T*)in, ld_in, \
                     (const T*)wq, (const T*)wk, cos_t, sin_t, (T*)out,       \
                     ld_out, rstd_q, rstd_k)
  if (dtype == 1) {
    if (d_h == 128) Q3L_QF(bf16_t, 128); else Q3L_QF(bf16_t, 64);
  } else {
    if (d_h == 128) Q3L_QF(float, 128); else Q3L_QF(float, 64);
  }
#undef Q3L_QF
  return hipGetLastError();
}

hipError_t qknorm_rope_bwd(int dtype, int B, int L, int h_q, int h_kv,
                           int d_h, int qk_norm, const void* g_in,
                           int64_t ld_g, const void* pre, int64_t ld_pre,
                           const void* wq, const void* wk, const float* rstd_q,
                           const float* rstd_k, const float* cos_t,
                           const float* sin_t, void* out, int64_t ld_out,
                           float* wq_part, float* wk_part, int* nparts,
                           hipStream_t s) {
  const int64_t tokens = (int64_t)B * L;
  // Each workgroup writes one partial row of the q/k norm weight gradients.
  const int64_t grid = qknorm_bwd_grid(tokens, h_q + h_kv, d_h);
  *nparts = (int)grid;
#define Q3L_QB(T, D)                                                            \
  hipLaunchKernelGGL((qknorm_rope_bwd_kernel<T, D>), dim3(grid), dim3(256), 0, s, \
                     tokens, L, h_q, h_kv, qk_norm, (const T*)g_in, ld_g,       \
                     (const T*)pre, ld_pre, (const T*)wq, (const T*)wk, rstd_q, \
                     rstd_k, cos_t, sin_t, (T*)out, ld_out, wq_part, wk_part)
  if (dtype == 1) {
    if (d_h == 128) Q3L_QB(bf16_t, 128); else Q3L_QB(bf16_t, 64);
  } else {
    if (d_h == 128) Q3L_QB(float, 128); else Q3L_QB(float, 64);
  }
#undef Q3L_QB
  return hipGetLastError();
}

}  // namespace q3l
