// The token embedding at the bottom of the model (walkthrough page, the
// "简化的 Qwen3 结构" listing: embed_tokens [vocab, d], tied with the output
// projection): the gather x[t] = E[ids[t]] and its adjoint, the scatter-add
// dE[v] += sum over the tokens t with ids[t] = v of dx[t].
//
// The scatter is deterministic, without atomics: a first kernel links every
// token to the next token with the same id and marks the first occurrence of
// each id (each workgroup stages the ids through LDS and every thread scans
// them for its own token); a second kernel gives each first occurrence one
// workgroup that walks its chain in token order and adds the rows once into
// dE.  Ids outside [0, V) gather zero rows and scatter nothing.
#include "common.h"
#include "ops.h"

namespace q3l {
namespace {

// One wave per token; 16-byte chunks of the row (row_bytes / 16 of them).
__global__ __launch_bounds__(256) void embed_gather_kernel(int64_t T, int64_t row_bytes, int V,
                                                           const int32_t* __restrict__ ids,
                                                           const char* __restrict__ E,
                                                           char* __restrict__ x) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int id = ids[t];
  const bool ok = id >= 0 && id < V;
  const char* src = E + (int64_t)(ok ? id : 0) * row_bytes;
  char* dst = x + t * row_bytes;
  for (int64_t c = lane; c < row_bytes / 16; c += 64)
    st16(dst + 16 * c, ok ? ld16(src + 16 * c) : u32x4_t{0u, 0u, 0u, 0u});
}

// next[t]: the smallest u > t with ids[u] == ids[t], else T; first[t]: 1 iff
// no u < t has the same id.  Ids are scanned in LDS chunks of kChunk.
constexpr int kChunk = 4096;
__global__ __launch_bounds__(256) void embed_links_kernel(int T, const int32_t* __restrict__ ids,
                                                          int32_t* __restrict__ next,
                                                          int32_t* __restrict__ first) {
  __shared__ int32_t sid[kChunk];
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int my = t < T ? ids[t] : 0;
  int nx = T;
  bool fst = true;
  for (int base = 0; base < T; base += kChunk) {
    const int n = min(kChunk, T - base);
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += 256) sid[i] = ids[base + i];
    __syncthreads();
    for (int i = 0; i < n; ++i) {
      const int u = base + i;
      if (sid[i] == my) {
        if (u < t) fst = false;
        else if (u > t && u < nx) nx = u;
      }
    }
  }
  if (t < T) {
    next[t] = nx;
    first[t] = fst ? 1 : 0;
  }
}

// One workgroup per token; only first occurrences work.  Thread c holds
// 4-element column chunks c, c + 256, ... (CPT of them).
template <class T_, int CPT>
__global__ __launch_bounds__(256) void embed_scatter_kernel(int T, int d, int V,
                                                            const int32_t* __restrict__ ids,
                                                            const int32_t* __restrict__ next,
                                                            const int32_t* __restrict__ first,
                                                            const T_* __restrict__ dx,
                                                            float* __restrict__ dE) {
  const int t = blockIdx.x;
  if (!first[t]) return;
  const int id = ids[t];
  if (id < 0 || id >= V) return;
  float acc[CPT][4];
#pragma unroll
  for (int c = 0; c < CPT; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[c][j] = 0.f;
  for (int u = t; u < T; u = next[u]) {
    const T_* row = dx + (int64_t)u * d;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int col = 4 * (threadIdx.x + 256 * c);
      if (col < d) {
        if constexpr (sizeof(T_) == 2) {
          const u32x2_t v = ld8(row + col);
          acc[c][0] += lo_f(v[0]); acc[c][1] += hi_f(v[0]);
          acc[c][2] += lo_f(v[1]); acc[c][3] += hi_f(v[1]);
        } else {
          const f32x4_t v = *reinterpret_cast<const f32x4_t*>(row + col);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[c][j] += v[j];
        }
      }
    }
  }
  float* out = dE + (int64_t)id * d;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int col = 4 * (threadIdx.x + 256 * c);
    if (col < d) {
      f32x4_t o = *reinterpret_cast<f32x4_t*>(out + col);
      o += f32x4_t{acc[c][0], acc[c][1], acc[c][2], acc[c][3]};
      *reinterpret_cast<f32x4_t*>(out + col) = o;
    }
  }
}

}  // namespace

hipError_t embed_gather(int dtype, int64_t T, int d, int V, const int32_t* ids, const void* E,
                        void* x, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int64_t rb = (int64_t)d * (dtype == 1 ? 2 : 4);
  hipLaunchKernelGGL(embed_gather_kernel, dim3((unsigned)cdiv(T, 4)), dim3(256), 0, s, T, rb, V,
                     ids, (const char*)E, (char*)x);
  return hipGetLastError();
}

hipError_t embed_scatter_add(int dtype, int T, int d, int V, const int32_t* ids,
                             const void* dx, int32_t* next, int32_t* first, float* dE,
                             hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(embed_links_kernel, dim3((unsigned)cdiv(T, 256)), dim3(256), 0, s, T, ids,
                     next, first);
  const int cpt = (int)cdiv(d, 4 * 256);
#define Q3L_ES(TY, C)                                                                 \
  hipLaunchKernelGGL((embed_scatter_kernel<TY, C>), dim3((unsigned)T), dim3(256), 0, s, T, d, \
                     V, ids, next, first, (const TY*)dx, dE)
#define Q3L_ES_ALL(TY)                  \
  if (cpt <= 1) Q3L_ES(TY, 1);          \
  else if (cpt <= 2) Q3L_ES(TY, 2);     \
  else if (cpt <= 4) Q3L_ES(TY, 4);     \
  else if (cpt <= 8) Q3L_ES(TY, 8);     \
  else return hipErrorInvalidValue;
  if (dtype == 1) {
    Q3L_ES_ALL(bf16_t)
  } else {
    Q3L_ES_ALL(float)
  }
#undef Q3L_ES_ALL
#undef Q3L_ES
  return hipGetLastError();
}

}  // namespace q3l
