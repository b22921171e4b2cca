// fp32 GEMM for the fp32 layer (the small fp32 workload): same operand /
// epilogue description as the bf16 matrix-core GEMM, evaluated one output
// element per thread with LDS-free fp32 FMAs.  Correctness path only.
#include "common.h"
#include "ops.h"

namespace q3l {
namespace {

__device__ inline int seg_of32(const int32_t* start, int nseg, int idx) {
  int s = 0;
  if (nseg > 1 && idx >= start[1]) s = 1;
  if (nseg > 2 && idx >= start[2]) s = 2;
  return s;
}

// Pointer to element (r, 0) of a K-contiguous operand, or element (r, k) of
// a row-contiguous one.
__device__ inline float opnd(const Operand& o, int r, int k) {
  if (o.k_contig) {
    if (o.paired) {
      const int seg = (r >> 5) & 1;
      const int rr = (r >> 6) * 32 + (r & 31);
      return static_cast<const float*>(o.p[seg])[(int64_t)rr * o.ld[seg] + k];
    }
    const int s = seg_of32(o.start, o.nseg, r);
    return static_cast<const float*>(o.p[s])[(int64_t)(r - o.start[s]) * o.ld[s] + k];
  }
  const int s = seg_of32(o.start, o.nseg, k);
  return static_cast<const float*>(o.p[s])[(int64_t)(k - o.start[s]) * o.ld[s] + r];
}

__device__ inline float dot_mk(const GemmArgs& g, int m, int n) {
  float acc = 0.f;
  for (int k = 0; k < g.K; ++k) acc += opnd(g.a, m, k) * opnd(g.b, n, k);
  return acc;
}

__global__ void gemm_f32_kernel(const GemmArgs g, int nbx) {
  const Epilogue& e = g.epi;
  const int m = blockIdx.x / nbx;
  const int bx = blockIdx.x % nbx;
  if (e.kind == EPI_SILU_MUL) {
    const int f = bx * blockDim.x + threadIdx.x;
    if (f >= e.ffn) return;
    const int rg = (f / 32) * 64 + (f % 32);
    const float gv = dot_mk(g, m, rg), uv = dot_mk(g, m, rg + 32);
    static_cast<float*>(e.c)[(int64_t)m * e.ldc + f] = gv / (1.0f + expf(-gv)) * uv;
    if (e.gu) {
      float* G = static_cast<float*>(e.gu) + (int64_t)m * e.ldgu;
      G[f] = gv;
      G[e.ffn + f] = uv;
    }
    return;
  }
  const int n = bx * blockDim.x + threadIdx.x;
  if (n >= g.N) return;
  const float v = dot_mk(g, m, n);
  switch (e.kind) {
    case EPI_STORE: {
      float o = v;
      if (e.r) o += static_cast<const float*>(e.r)[(int64_t)m * e.ldr + n];
      static_cast<float*>(e.c)[(int64_t)m * e.ldc + n] = o;
      break;
    }
    case EPI_PARTIAL:
      e.p32[(int64_t)m * e.ldp + n] = v;
      if (e.c)
        static_cast<float*>(e.c)[(int64_t)m * e.ldc + n] =
            v + static_cast<const float*>(e.r)[(int64_t)m * e.ldr + n];
      break;
    case EPI_SILU_BWD: {
      const float* G = static_cast<const float*>(e.r) + (int64_t)m * e.ldr;
      const float gv = G[n], uv = G[e.ffn + n];
      const float sg = 1.0f / (1.0f + expf(-gv));
      float* D = static_cast<float*>(e.c) + (int64_t)m * e.ldc;
      D[n] = v * uv * sg * (1.0f + gv * (1.0f - sg));
      D[e.ffn + n] = v * gv * sg;
      break;
    }
    case EPI_WGRAD: {
      const int s = seg_of32(e.cstart, e.cnseg, m);
      float* C = e.cs[s] + (int64_t)(m - e.cstart[s]) * e.ldc + n;
      *C = e.accumulate ? *C + v : v;
      break;
    }
    default:
      break;
  }
}

}  // namespace

hipError_t gemm_f32(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.K <= 0) return hipSuccess;
  const int width = g.epi.kind == EPI_SILU_MUL ? g.epi.ffn : g.N;
  const int nbx = (int)cdiv(width, 128);
  dim3 grid((unsigned)((int64_t)nbx * g.M)), block(128);
  hipLaunchKernelGGL(gemm_f32_kernel, grid, block, 0, s, g, nbx);
  return hipGetLastError();
}

}  // namespace q3l
