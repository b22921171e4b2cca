// bf16 transpose, dst[c][r] = src[r][c], used by the layer's backward to put
// every GEMM operand in K-contiguous form (the matrix-core kernel's fastest
// layout).  HBM-bound: each lane moves one 8x8 block through registers
// (8 loads of 16 bytes, an in-register transpose, 8 stores of 16 bytes); a
// wave covers a 64x64 tile with lanes arranged so that every load and every
// store instruction touches 128 contiguous bytes per row.  No LDS.
#include "common.h"
#include "ops.h"

namespace q3l {
namespace {

// rows_pad >= rows, both and cols multiples of 8 except rows (any); columns
// r in [rows, rows_pad) of dst are written as zeros.
__global__ __launch_bounds__(256) void transpose_kernel(
    int rows, int rows_pad, int cols, const bf16_t* __restrict__ src, int64_t lds,
    bf16_t* __restrict__ dst, int64_t ldd) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int ntc = (cols + 63) / 64;
  const int64_t tr = wid / ntc;
  const int tc = (int)(wid % ntc);
  const int a = lane & 7, b = lane >> 3;
  const int64_t r0 = tr * 64 + 8 * a;
  const int c0 = tc * 64 + 8 * b;
  if (r0 >= rows_pad || c0 >= cols) return;
  u32x4_t in[8], out[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int64_t rr = r0 + r;
    in[r] = rr < rows ? ld16(src + rr * lds + c0) : u32x4_t{0u, 0u, 0u, 0u};
  }
  transpose8x8(in, out);
#pragma unroll
  for (int c = 0; c < 8; ++c) st16(dst + (int64_t)(c0 + c) * ldd + r0, out[c]);
}

}  // namespace

hipError_t transpose_bf16(int rows, int rows_pad, int cols, const void* src,
                          int64_t ld_src, void* dst, int64_t ld_dst, hipStream_t s) {
  if (rows_pad <= 0 || cols <= 0) return hipSuccess;
  const int64_t tiles = cdiv(rows_pad, 64) * cdiv(cols, 64);
  hipLaunchKernelGGL(transpose_kernel, dim3((unsigned)cdiv(tiles, 4)), dim3(256), 0, s,
                     rows, rows_pad, cols, (const bf16_t*)src, ld_src, (bf16_t*)dst,
                     ld_dst);
  return hipGetLastError();
}

}  // namespace q3l
