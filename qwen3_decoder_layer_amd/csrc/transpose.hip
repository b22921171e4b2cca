// bf16 transpose, dst[c][r] = src[r][c], used by the layer's backward to put
// every GEMM operand in K-contiguous form (the matrix-core kernel's fastest
// layout); several transposes go out as one launch, so the small ones do
// not each pay a launch's ramp-up and tail.  HBM-bound: each lane moves one 8x8 block through registers
// (8 loads of 16 bytes, an in-register transpose, 8 stores of 16 bytes); a
// wave covers a 64x64 tile with lanes arranged so that every load and every
// store instruction touches 128 contiguous bytes per row.  No LDS.
#include "common.h"
#include "ops.h"

namespace q3l {
namespace {

// One transpose of a batch: rows_pad >= rows, cols and rows_pad multiples of
// 8 (rows any); columns r in [rows, rows_pad) of dst are written as zeros.
// Workgroups first_wg .. (next job's first_wg) - 1 cover it, 4 tiles each.
struct TransposeBatch {
  int n;
  int first_wg[kTransposeBatchMax + 1];
  TransposeJob job[kTransposeBatchMax];
};

__global__ __launch_bounds__(256) void transpose_kernel(const TransposeBatch b) {
  // Which job: a uniform scan over at most kTransposeBatchMax entries.
  const int bid = blockIdx.x;
  int jx = 0;
#pragma unroll
  for (int i = 1; i < kTransposeBatchMax; ++i) jx += (i < b.n && bid >= b.first_wg[i]) ? 1 : 0;
  const TransposeJob& J = b.job[jx];
  const int rows = J.rows, rows_pad = J.rows_pad, cols = J.cols;
  const bf16_t* __restrict__ src = static_cast<const bf16_t*>(J.src);
  bf16_t* __restrict__ dst = static_cast<bf16_t*>(J.dst);
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)(bid - b.first_wg[jx]) * 4 + (threadIdx.x >> 6);
  const int ntc = (cols + 63) / 64;
  const int64_t tr = wid / ntc;
  const int tc = (int)(wid % ntc);
  const int a = lane & 7, bb = lane >> 3;
  const int64_t r0 = tr * 64 + 8 * a;
  const int c0 = tc * 64 + 8 * bb;
  if (r0 >= rows_pad || c0 >= cols) return;
  u32x4_t in[8], out[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int64_t rr = r0 + r;
    in[r] = rr < rows ? ld16(src + rr * J.ld_src + c0) : u32x4_t{0u, 0u, 0u, 0u};
  }
  transpose8x8(in, out);
#pragma unroll
  for (int c = 0; c < 8; ++c) st16(dst + (int64_t)(c0 + c) * J.ld_dst + r0, out[c]);
}

}  // namespace

hipError_t transpose_bf16_batch(const TransposeJob* jobs, int n, hipStream_t s) {
  if (n < 0 || n > kTransposeBatchMax) return hipErrorInvalidValue;
  TransposeBatch b{};
  int64_t wg = 0;
  for (int i = 0; i < n; ++i) {
    const TransposeJob& j = jobs[i];
    b.first_wg[b.n] = (int)wg;
    if (j.rows_pad <= 0 || j.cols <= 0) continue;
    b.job[b.n++] = j;
    wg += cdiv(cdiv(j.rows_pad, 64) * cdiv(j.cols, 64), 4);
  }
  b.first_wg[b.n] = (int)wg;
  if (wg == 0) return hipSuccess;
  if (wg > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(transpose_kernel, dim3((unsigned)wg), dim3(256), 0, s, b);
  return hipGetLastError();
}

hipError_t transpose_bf16(int rows, int rows_pad, int cols, const void* src,
                          int64_t ld_src, void* dst, int64_t ld_dst, hipStream_t s) {
  const TransposeJob j{src, ld_src, dst, ld_dst, rows, rows_pad, cols};
  return transpose_bf16_batch(&j, 1, s);
}

}  // namespace q3l
