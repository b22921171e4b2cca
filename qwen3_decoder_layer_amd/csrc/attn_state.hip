// Merging and finishing the block states of attention (the parallelism page,
// section 4.2, ring attention): for one query and one block of keys the
// state is (m, l, acc) -- the block's largest scaled score, l = sum of
// exp(s - m) and acc = sum of exp(s - m) v.  Two states are merged by scaling
// each one's l and acc by exp(m_i - m_new), m_new = max(m_1, m_2), and adding;
// the output is acc / l and the log-sum-exp m + log l.  A state of a query
// that saw no key in its block is (-inf, 0, 0) and drops out of a merge.
//
// Both kernels are elementwise and HBM-bound: one thread per 4 elements of a
// (token, head) row, 16-byte accesses; m and l are read (and written) once
// per row by the row's first thread.
#include "common.h"
#include "ops.h"

namespace q3l {
namespace {

__global__ __launch_bounds__(256) void attn_merge_kernel(int B, int L, int h_q, int d_h,
                                                         float* __restrict__ m,
                                                         float* __restrict__ l,
                                                         float* __restrict__ acc,
                                                         const float* __restrict__ m2,
                                                         const float* __restrict__ l2,
                                                         const float* __restrict__ acc2) {
  const int per_row = d_h / 4;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rows = (int64_t)B * L * h_q;
  if (i >= rows * per_row) return;
  const int64_t row = i / per_row;          // (token, head), token-major
  const int c = (int)(i % per_row);
  const int head = (int)(row % h_q);
  const int64_t tok = row / h_q;
  const int b = (int)(tok / L), t = (int)(tok % L);
  const int64_t si = ((int64_t)b * h_q + head) * L + t;
  const float ma = m[si], mb = m2[si];
  const float mn = fmaxf(ma, mb);
  const float fa = ma == -INFINITY ? 0.f : expf(ma - mn);
  const float fb = mb == -INFINITY ? 0.f : expf(mb - mn);
  const int64_t off = tok * (int64_t)h_q * d_h + (int64_t)head * d_h + 4 * c;
  const f32x4_t a = *reinterpret_cast<const f32x4_t*>(acc + off);
  const f32x4_t b2 = *reinterpret_cast<const f32x4_t*>(acc2 + off);
  *reinterpret_cast<f32x4_t*>(acc + off) = a * fa + b2 * fb;
  if (c == 0) {
    l[si] = l[si] * fa + l2[si] * fb;
    m[si] = mn;
  }
}

template <class T>
__global__ __launch_bounds__(256) void attn_finish_kernel(int B, int L, int h_q, int d_h,
                                                          const float* __restrict__ m,
                                                          const float* __restrict__ l,
                                                          const float* __restrict__ acc,
                                                          T* __restrict__ o, int64_t ldo,
                                                          float* __restrict__ lse) {
  const int per_row = d_h / 4;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rows = (int64_t)B * L * h_q;
  if (i >= rows * per_row) return;
  const int64_t row = i / per_row;
  const int c = (int)(i % per_row);
  const int head = (int)(row % h_q);
  const int64_t tok = row / h_q;
  const int b = (int)(tok / L), t = (int)(tok % L);
  const int64_t si = ((int64_t)b * h_q + head) * L + t;
  const float lv = l[si];
  const float inv = lv > 0.f ? 1.0f / lv : 0.f;
  const f32x4_t a = *reinterpret_cast<const f32x4_t*>(
      acc + tok * (int64_t)h_q * d_h + (int64_t)head * d_h + 4 * c);
  T* op = o + tok * ldo + (int64_t)head * d_h + 4 * c;
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<u32x2_t*>(op) = u32x2_t{pack2(a[0] * inv, a[1] * inv),
                                              pack2(a[2] * inv, a[3] * inv)};
  } else {
    *reinterpret_cast<f32x4_t*>(op) = a * inv;
  }
  if (c == 0) lse[si] = lv > 0.f ? m[si] + logf(lv) : -INFINITY;
}

}  // namespace

hipError_t attn_state_merge(int B, int L, int h_q, int d_h, float* m, float* l, float* acc,
                            const float* m2, const float* l2, const float* acc2,
                            hipStream_t s) {
  const int64_t n = (int64_t)B * L * h_q * (d_h / 4);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, B, L,
                     h_q, d_h, m, l, acc, m2, l2, acc2);
  return hipGetLastError();
}

hipError_t attn_state_finish(int dtype, int B, int L, int h_q, int d_h, const float* m,
                             const float* l, const float* acc, void* o, int64_t ldo,
                             float* lse, hipStream_t s) {
  const int64_t n = (int64_t)B * L * h_q * (d_h / 4);
  if (n <= 0) return hipSuccess;
  if (dtype == 1)
    hipLaunchKernelGGL((attn_finish_kernel<bf16_t>), dim3((unsigned)cdiv(n, 256)), dim3(256),
                       0, s, B, L, h_q, d_h, m, l, acc, (bf16_t*)o, ldo, lse);
  else
    hipLaunchKernelGGL((attn_finish_kernel<float>), dim3((unsigned)cdiv(n, 256)), dim3(256),
                       0, s, B, L, h_q, d_h, m, l, acc, (float*)o, ldo, lse);
  return hipGetLastError();
}

}  // namespace q3l
