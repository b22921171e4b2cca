// SwiGLU adjoint (walkthrough page, Step 9: f = silu(g) * u with
// g = hn W_gate^T, u = hn W_up^T), bf16, fused with the transposed copy the
// gate/up weight-gradient GEMM reads:
//   dg = df * u * s * (1 + g (1 - s)),  du = df * g * s,   s = sigmoid(g)
// written to dgu = [dg | du] ([T, 2 ffn], row-major) and, when asked, to
// dguT = [dg | du]^T ([2 ffn, Tp]); the transposed columns t >= T are zero.
// A second form writes only the transposed copy, from a dgu an earlier pass
// left (the weight-gradient half of a split backward): bitwise what the
// fused form writes.
// HBM-bound: each lane moves one 8x8 block of df, g and u through registers
// (16-byte loads), and writes its 8x8 blocks of dg and du as rows and (after
// an in-register transpose) as columns.  A wave covers 64 tokens x 64
// features; every load and store instruction touches 128 contiguous bytes
// per row.  dgu's dg half may hold df itself: each lane reads its df block
// before writing the dg block at the same place.
// The fp32 form (the correctness path's phase entry) is plain elementwise
// code.
#include "common.h"
#include "ops.h"

namespace q3l {
namespace {

__device__ inline float sigmoid_f(float g) { return __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

template <bool FROM_DGU>
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(
    int T, int Tp, int ffn, const bf16_t* df, int64_t ld_df, const bf16_t* gu,
    int64_t ld_gu, bf16_t* dgu, int64_t ld_dgu, bf16_t* dguT, int64_t ld_t) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int ntc = (ffn + 63) / 64;
  const int64_t tr = wid / ntc;
  const int tc = (int)(wid % ntc);
  const int a = lane & 7, b = lane >> 3;
  const int64_t t0 = tr * 64 + 8 * a;
  const int f0 = tc * 64 + 8 * b;
  if (t0 >= Tp || f0 >= ffn) return;
  u32x4_t og[8], ou[8];
  if constexpr (FROM_DGU) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int64_t t = t0 + r;
      const bool ok = t < T;
      const u32x4_t z{0u, 0u, 0u, 0u};
      og[r] = ok ? ld16(dgu + t * ld_dgu + f0) : z;
      ou[r] = ok ? ld16(dgu + t * ld_dgu + ffn + f0) : z;
    }
  } else {
    u32x4_t vd[8], vg[8], vu[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int64_t t = t0 + r;
      const bool ok = t < T;
      const u32x4_t z{0u, 0u, 0u, 0u};
      vd[r] = ok ? ld16(df + t * ld_df + f0) : z;
      vg[r] = ok ? ld16(gu + t * ld_gu + f0) : z;
      vu[r] = ok ? ld16(gu + t * ld_gu + ffn + f0) : z;
    }
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float g0 = lo_f(vg[r][w]), g1 = hi_f(vg[r][w]);
        const float u0 = lo_f(vu[r][w]), u1 = hi_f(vu[r][w]);
        const float s0 = sigmoid_f(g0), s1 = sigmoid_f(g1);
        const float d0 = lo_f(vd[r][w]), d1 = hi_f(vd[r][w]);
        og[r][w] = pack2(d0 * u0 * s0 * (1.0f + g0 * (1.0f - s0)),
                         d1 * u1 * s1 * (1.0f + g1 * (1.0f - s1)));
        ou[r][w] = pack2(d0 * g0 * s0, d1 * g1 * s1);
      }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int64_t t = t0 + r;
      if (t < T) {
        st16(dgu + t * ld_dgu + f0, og[r]);
        st16(dgu + t * ld_dgu + ffn + f0, ou[r]);
      }
    }
  }
  if (dguT == nullptr) return;
  u32x4_t tg[8], tu[8];
  transpose8x8(og, tg);
  transpose8x8(ou, tu);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    st16(dguT + (int64_t)(f0 + c) * ld_t + t0, tg[c]);
    st16(dguT + (int64_t)(ffn + f0 + c) * ld_t + t0, tu[c]);
  }
}

// fp32: one thread per (token, feature).
__global__ __launch_bounds__(256) void swiglu_bwd_f32_kernel(
    int64_t M, int ffn, const float* df, int64_t ld_df, const float* gu, int64_t ld_gu,
    float* dgu, int64_t ld_dgu) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= M * ffn) return;
  const int64_t t = i / ffn;
  const int f = (int)(i % ffn);
  const float d = df[t * ld_df + f], g = gu[t * ld_gu + f], u = gu[t * ld_gu + ffn + f];
  const float s = 1.0f / (1.0f + expf(-g));
  dgu[t * ld_dgu + f] = d * u * s * (1.0f + g * (1.0f - s));
  dgu[t * ld_dgu + ffn + f] = d * g * s;
}

}  // namespace

hipError_t swiglu_bwd_f32(int64_t M, int ffn, const float* df, int64_t ld_df, const float* gu,
                          int64_t ld_gu, float* dgu, int64_t ld_dgu, hipStream_t s) {
  if (M <= 0 || ffn <= 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_bwd_f32_kernel, dim3((unsigned)cdiv(M * ffn, 256)), dim3(256), 0,
                     s, M, ffn, df, ld_df, gu, ld_gu, dgu, ld_dgu);
  return hipGetLastError();
}

hipError_t swiglu_transposes_bf16(int T, int Tp, int ffn, const void* dgu, int64_t ld_dgu,
                                  void* dguT, int64_t ld_t, hipStream_t s) {
  if (Tp <= 0 || ffn <= 0) return hipSuccess;
  const int64_t tiles = cdiv(Tp, 64) * cdiv(ffn, 64);
  hipLaunchKernelGGL(swiglu_bwd_kernel<true>, dim3((unsigned)cdiv(tiles, 4)), dim3(256), 0, s,
                     T, Tp, ffn, (const bf16_t*)nullptr, (int64_t)0, (const bf16_t*)nullptr,
                     (int64_t)0, (bf16_t*)const_cast<void*>(dgu), ld_dgu, (bf16_t*)dguT, ld_t);
  return hipGetLastError();
}

hipError_t swiglu_bwd_bf16(int T, int Tp, int ffn, const void* df, int64_t ld_df,
                           const void* gu, int64_t ld_gu, void* dgu, int64_t ld_dgu,
                           void* dguT, int64_t ld_t, hipStream_t s) {
  if (Tp <= 0 || ffn <= 0) return hipSuccess;
  const int64_t tiles = cdiv(Tp, 64) * cdiv(ffn, 64);
  hipLaunchKernelGGL(swiglu_bwd_kernel<false>, dim3((unsigned)cdiv(tiles, 4)), dim3(256), 0, s,
                     T, Tp, ffn, (const bf16_t*)df, ld_df, (const bf16_t*)gu, ld_gu,
                     (bf16_t*)dgu, ld_dgu, (bf16_t*)dguT, ld_t);
  return hipGetLastError();
}

}  // namespace q3l
