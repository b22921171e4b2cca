// Shared device-side helpers for the gfx950 kernels: bf16 conversion, vector
// types, MFMA wrappers, wave reductions and the in-register 8x8 transpose.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q3l {

typedef uint16_t bf16_t;  // raw bfloat16 bits

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// ---- bf16 <-> fp32 ---------------------------------------------------------
__host__ __device__ inline float bf2f(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// fp32 -> bf16, round to nearest (ties to even): one v_cvt_pk_bf16_f32 per
// pair of values on gfx950.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pack2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
__device__ inline bf16_t f2bf(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}
__host__ __device__ inline float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__host__ __device__ inline float hi_f(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---- generic element access for the fp32 / bf16 kernels --------------------
template <class T> struct Elem;
template <> struct Elem<float> {
  __device__ static inline float load(const float* p) { return *p; }
  __device__ static inline void store(float* p, float v) { *p = v; }
};
template <> struct Elem<bf16_t> {
  __device__ static inline float load(const bf16_t* p) { return bf2f(*p); }
  __device__ static inline void store(bf16_t* p, float v) { *p = f2bf(v); }
};

// ---- 16-byte global / LDS moves -------------------------------------------
__device__ inline u32x4_t ld16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}
__device__ inline void st16(void* p, u32x4_t v) {
  *reinterpret_cast<u32x4_t*>(p) = v;
}
__device__ inline u32x2_t ld8(const void* p) {
  return *reinterpret_cast<const u32x2_t*>(p);
}
__device__ inline void st8(void* p, u32x2_t v) {
  *reinterpret_cast<u32x2_t*>(p) = v;
}

// ---- 8x8 transpose of 16-bit elements held as 8 rows of 4 dwords ----------
// in[r] holds elements (r, 0..7) (two per dword, low half first); out[c]
// receives elements (0..7, c).
__host__ __device__ inline void transpose8x8(const u32x4_t in[8], u32x4_t out[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t a = in[2 * j][c >> 1];
      const uint32_t b = in[2 * j + 1][c >> 1];
      out[c][j] = (c & 1) ? ((a >> 16) | (b & 0xFFFF0000u))
                          : ((a & 0xFFFFu) | (b << 16));
    }
  }
}

// ---- MFMA wrappers ---------------------------------------------------------
// mfma32(a, b, c): D[r][col] += sum_k A[r][k] B[k][col] for a 32x32x16 bf16
// tile.  Lane l supplies A[l%32][8*(l/32)+j] in a[j] and B[8*(l/32)+j][l%32]
// in b[j]; it receives D[8*(i/4) + 4*(l/32) + i%4][l%32] in d[i].
__device__ inline f32x16_t mfma32(const u32x4_t& a, const u32x4_t& b,
                                  const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
      __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0,
      0, 0);
}
// mfma16(a, b, c): the same for a 16x16x32 bf16 tile.  Lane l supplies
// A[l%16][8*(l/16)+j] in a[j] and B[8*(l/16)+j][l%16] in b[j]; it receives
// D[4*(l/16) + i][l%16] in d[i].
__device__ inline f32x4_t mfma16(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
      __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0,
      0, 0);
}

// ---- wave reductions (wave64) ---------------------------------------------
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// Sum over aligned groups of `width` lanes (width a power of two <= 64).
__device__ inline float group_sum(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) {
  return (a + b - 1) / b;
}

// Consecutive workgroup ids of a launch go round-robin to the 8 XCDs (each
// with its own L2).  Renumbered so XCD x works through one contiguous range
// of the nb logical ids, in order: the logical id of workgroup bid.
__device__ inline int xcd_contiguous(int bid, int nb) {
  const int xcd = bid & 7, slot = bid >> 3;
  const int per = nb >> 3, rem = nb & 7;
  return (xcd < rem) ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

// ---- LDS: direct loads from global memory and transposing reads ----------
#define Q3L_LDS __attribute__((address_space(3)))
#define Q3L_GLOBAL __attribute__((address_space(1)))

__device__ inline uint32_t uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ inline uint64_t uni64(uint64_t v) {
  return ((uint64_t)uni((uint32_t)(v >> 32)) << 32) | uni((uint32_t)v);
}
__device__ inline uint32_t lds_addr(const Q3L_LDS void* p) {
  return (uint32_t)(uintptr_t)p;
}

constexpr uint32_t kOOB = 0x80000000u;   // any offset past the buffer range

// Global -> LDS without registers: lane i's 16 (lds_dma16) or 4 (lds_dma4)
// bytes land at LDS byte lds_base + 16 i (4 i); lds_base is uniform.  The
// buffer covers [p, p + 2 GiB) with stride 0, so `voff + soff` (per-lane +
// uniform) is a byte offset and an offset >= 2^31 (kOOB) reads zeros.  These
// writes are counted by vmcnt; a kernel orders them against its own LDS
// reads with an explicit s_waitcnt vmcnt and a barrier.
//
// The instruction is written in inline assembly (M0 = LDS base, one wait
// state, then buffer_load ... lds).  Issued through the compiler's builtin,
// it makes the compiler put an s_waitcnt vmcnt(0) in front of every later
// transposing LDS read (ds_read_b64_tr_b16), whatever address that reads:
// each loop iteration would then wait, mid-iteration, for the prefetch it
// has just issued.  The assembly form has no register results, so nothing
// is left in flight towards a register the compiler could reuse, and the
// compiler's own vmcnt counts (for its register loads) only over-wait, as
// loads complete in issue order.
__device__ inline void lds_dma16_r(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                   uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(r), "s"(soff), "s"(lds_base) : "memory", "m0");
}
// The same with the non-temporal policy: for data read once (it streams
// through the caches instead of displacing what other waves re-read).
__device__ inline void lds_dma16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                   uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen nt lds"
               :: "v"(voff), "s"(r), "s"(soff), "s"(lds_base) : "memory", "m0");
}
__device__ inline void lds_dma16(uint64_t p, uint32_t voff, uint32_t soff, uint32_t lds_base) {
  lds_dma16_r(__builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, 0x7FFFFFFF, 0x00020000),
              voff, soff, lds_base);
}
__device__ inline void lds_dma4(uint64_t p, uint32_t voff, uint32_t lds_base) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, 0x7FFFFFFF, 0x00020000);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :: "v"(voff), "s"(r), "s"(lds_base) : "memory", "m0");
}

// Buffer resource over [p, p + bytes) (bytes 0: every access is out of
// range) and 16- / 4-byte accesses through it at a per-lane byte offset.
// Out-of-range loads (offset kOOB) return zeros and out-of-range stores are
// dropped, so bounds need no branches.
__device__ inline __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, uint32_t bytes = 0x7FFFFFFFu) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ inline u32x4_t buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ inline float buf_ldf(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
// Cache-policy bit of a buffer access: non-temporal (streamed past the
// caches' retention).
constexpr int kNT = 2;
template <int AUX = 0>
__device__ inline void buf_st16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, AUX);
}
__device__ inline u32x2_t buf_ld8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
template <int AUX = 0>
__device__ inline void buf_st8(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2_t v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(decltype(
      __builtin_amdgcn_raw_buffer_load_b64(r, 0, 0, 0)), v), r, off, 0, AUX);
}

template <int N>
__device__ inline void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Workgroup barrier for LDS stages: this wave's LDS reads have returned (so
// a stage it read may be refilled once everyone is past), without the
// vmcnt(0) a fenced __syncthreads() would add -- direct loads of younger
// stages stay in flight.  The memory clobber keeps LDS accesses on their
// side of it.
__device__ inline void stage_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ inline u32x4_t ld_lds16(const Q3L_LDS void* p) {
  return *reinterpret_cast<const Q3L_LDS u32x4_t*>(p);
}
// Transposing 8-byte LDS read of 16-bit elements (ds_read_b64_tr_b16).  In
// each 16-lane group, output lane j receives element (j % 4) of the 8 bytes
// addressed by source lanes 4e + j / 4, e = 0..3, as its element e.
typedef short i16x4_t __attribute__((ext_vector_type(4)));
__device__ inline u32x2_t ld_tr8(const Q3L_LDS void* p) {
  return __builtin_bit_cast(
      u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((Q3L_LDS i16x4_t*)(p)));
}
// Two transposing reads (at p and p + second bytes) forming one MFMA operand.
__device__ inline u32x4_t ld_tr_pair(const Q3L_LDS void* p, int second) {
  const u32x2_t a = ld_tr8(p);
  const u32x2_t b = ld_tr8((const Q3L_LDS char*)p + second);
  return u32x4_t{a[0], a[1], b[0], b[1]};
}

}  // namespace q3l
