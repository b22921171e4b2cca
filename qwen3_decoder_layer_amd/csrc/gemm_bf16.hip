// bf16 GEMM on the gfx950 matrix cores for the seven projections of the
// Qwen3 decoder layer (walkthrough page, Steps 2, 6 and 9) and their
// input/weight gradients.
//
// C[M, N] = sum_k A(m, k) B(n, k), fp32 accumulation.
//
// Design (one workgroup = 4 wave64s = one BM x BN output tile):
//  - K is consumed in slabs of KB (64).  A K-contiguous operand (activations
//    [T, f], weights [out, in]) goes from HBM straight into LDS with buffer
//    loads (buffer_load_dwordx4 ... lds): no staging registers, no LDS store
//    instructions.  Each wave-instruction fills 1 KiB of LDS, lane i the
//    i-th 16 bytes; lanes pick the global chunk that belongs at their
//    position.  Out-of-range k (the K tail) uses an offset past the buffer's
//    range, which the hardware returns as zero.
//  - An operand contiguous along its rows instead (a weight read as
//    [in, out], activations read along the token axis) is also loaded
//    straight into LDS, as it is in memory, and read with the gfx950
//    transposing LDS read (ds_read_b64_tr_b16).  That read sustains about a
//    third of ds_read_b128's byte rate, so the layer's backward transposes
//    its GEMM operands once (transpose.hip) and uses the K-contiguous path;
//    the transposed-read path serves the stand-alone gradient entry points.
//  - K-contiguous LDS tiles are [rows][KB] with the 16-byte chunks of row r XOR-swizzled
//    by (r >> 1) & 7, so the 16-byte fragment reads of 16 consecutive rows
//    hit 16 distinct bank groups.  Two LDS stages: the next slab streams in
//    while the matrix cores work on the current one; one barrier per slab.
//    Within a slab the next k-step's fragment reads are interleaved with
//    the current step's matrix instructions (scheduling-group barriers).
//  - The waves form a 2 x 2 grid; each owns a (BM/2) x (BN/2) sub-tile of
//    32x32 accumulators (v_mfma_f32_32x32x16_bf16).  The B fragment is
//    passed as the MFMA's first operand so each lane ends up holding four
//    consecutive output columns of one row: epilogue stores are 8 or 16
//    bytes wide.
//  - Workgroup ids are renumbered so each of the 8 XCDs (own L2) receives a
//    contiguous range of tiles, and tiles are walked in groups of 8 tile
//    rows so concurrently running tiles share A and B panels in L2.
//  - Fused epilogues: residual add (Steps 7 and 10), fp32 partial output for
//    a tensor-parallel share, silu(gate) * up over an interleaved gate/up
//    operand (Step 9), the SwiGLU backward, and fp32 (+=) weight gradients.
#include "common.h"
#include "ops.h"

namespace q3l {
namespace {

constexpr uint32_t kOOB = 0x80000000u;   // any offset past the buffer range

#define Q3L_LDS __attribute__((address_space(3)))

__device__ inline uint32_t uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ inline uint64_t uni64(uint64_t v) {
  return ((uint64_t)uni((uint32_t)(v >> 32)) << 32) | uni((uint32_t)v);
}

// 16 bytes per lane from a raw buffer straight into LDS: lane i's data lands
// at LDS byte lds_base + 16 * i.  The buffer covers [p, p + 2 GiB) with
// stride 0, so `voff` is a byte offset and any offset >= 2^31 reads zeros.
// Issued as inline asm: the compiler then does not treat the pending LDS
// writes as aliasing every LDS read of the current slab (it would otherwise
// wait for the next slab's loads before reading this one).  The kernel waits
// for these loads itself (s_waitcnt vmcnt(0) before each slab's barrier).
typedef uint32_t u32x4s_t __attribute__((ext_vector_type(4)));
__device__ inline void dma16(uint64_t p, uint32_t voff, uint32_t lds_base) {
  const u32x4s_t rsrc = {(uint32_t)p, (uint32_t)(p >> 32) & 0xFFFFu, 0x7FFFFFFFu,
                         0x00020000u};
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(rsrc), "s"(lds_base)
      : "memory", "m0");
}
__device__ inline uint32_t lds_addr(const Q3L_LDS char* p) {
  return (uint32_t)(uintptr_t)p;
}

// Segment holding index idx of an operand (idx uniform): base pointer, ld
// (elements) and start.  Every field is read from the kernel argument through
// readfirstlane before the select, so the compiler keeps the choice between
// register values instead of folding it into an indexed load of the table.
__device__ inline void pick(const Operand& o, int idx, uint64_t& p, int64_t& ld, int& st) {
  const int n = (int)uni((uint32_t)o.nseg);
  const int s1 = n > 1 ? (int)uni((uint32_t)o.start[1]) : 0x7fffffff;
  const int s2 = n > 2 ? (int)uni((uint32_t)o.start[2]) : 0x7fffffff;
  const uint64_t p0 = uni64((uint64_t)o.p[0]);
  const uint64_t p1 = uni64((uint64_t)o.p[n > 1 ? 1 : 0]);
  const uint64_t p2 = uni64((uint64_t)o.p[n > 2 ? 2 : 0]);
  const int64_t l0 = (int64_t)uni64((uint64_t)o.ld[0]);
  const int64_t l1 = (int64_t)uni64((uint64_t)o.ld[n > 1 ? 1 : 0]);
  const int64_t l2 = (int64_t)uni64((uint64_t)o.ld[n > 2 ? 2 : 0]);
  const bool b1 = idx >= s1, b2 = idx >= s2;
  p = b2 ? p2 : (b1 ? p1 : p0);
  ld = b2 ? l2 : (b1 ? l1 : l0);
  st = b2 ? s2 : (b1 ? s1 : 0);
}

// ---- K-contiguous operand: [R rows][KB k] in LDS --------------------------
// A row is KB*2 bytes = CPRK 16-byte chunks.  Wave-instruction q (= 4*i +
// wave) fills rows RPW*q .. RPW*q + RPW-1; lane l writes row RPW*q + l/CPRK,
// slot l%CPRK, holding global chunk (slot ^ swz(row)) of that row.  The
// swizzle makes the fragment reads of 16 consecutive rows (same chunk)
// conflict-free: KB=64: (row >> 1) & 7; KB=32: (row >> 2) & 3.
template <int KB>
__device__ inline int kswz(int row) {
  return KB == 64 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}

template <int R, int KB>
struct KOperand {
  static constexpr int CPRK = KB / 8;
  static constexpr int RPW = 64 / CPRK;
  static constexpr int NI = R / (4 * RPW);   // wave-instructions per thread per slab
  uint32_t voff[NI];   // per lane: byte offset of its chunk at k = 0
  int kel[NI];         // per lane: first k (elements) of its chunk at k0 = 0
  uint64_t base[NI];   // uniform: segment base of the instruction's rows

  __device__ void init(const Operand& o, int r0, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int q = 4 * i + wave;
      const int row = RPW * q + lane / CPRK;
      const int c = (lane % CPRK) ^ kswz<KB>(row);
      kel[i] = 8 * c;
      int gr = r0 + row;
      uint64_t p;
      int64_t ld;
      int st;
      if (o.paired) {
        const int g0 = r0 + RPW * q;        // uniform: first logical row
        const bool up = (g0 >> 5) & 1;
        const uint64_t pg = uni64((uint64_t)o.p[0]), pu = uni64((uint64_t)o.p[1]);
        const int64_t lg = (int64_t)uni64((uint64_t)o.ld[0]);
        const int64_t lu = (int64_t)uni64((uint64_t)o.ld[1]);
        p = up ? pu : pg;
        ld = up ? lu : lg;
        int pr = (gr >> 6) * 32 + (gr & 31);
        if (pr >= o.rows) pr = o.rows - 1;
        voff[i] = (uint32_t)((int64_t)pr * ld * 2 + 16 * c);
      } else {
        int g0 = r0 + RPW * q;
        if (g0 > o.rows - 1) g0 = o.rows - 1;
        pick(o, g0, p, ld, st);
        if (gr > o.rows - 1) gr = o.rows - 1;
        voff[i] = (uint32_t)((int64_t)(gr - st) * ld * 2 + 16 * c);
      }
      base[i] = p;
    }
  }
  // Issue the slab starting at k0 into LDS stage `dst` (R * KB * 2 bytes).
  __device__ void issue(const Operand&, int k0, int K, Q3L_LDS char* dst,
                        int wave) const {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint32_t off = (k0 + kel[i] < K) ? voff[i] + 2u * (uint32_t)k0 : kOOB;
      dma16(base[i], off, uni(lds_addr(dst + 1024 * (4 * i + wave))));
    }
  }
};

// ---- row-contiguous operand: [KB k][R] in LDS, read transposed -------------
// Element (r, k) at p[(k - start) * ld + r] (a weight read as [in, out], or
// activations read along the token axis).  The tile sits in LDS as in
// memory, [KB][R]: CPR 16-byte chunks per k-row; wave-instruction q fills
// k-rows RPI*q ..; lane l writes k-row RPI*q + l/CPR, slot l%CPR, holding
// global chunk slot ^ (4 * (krow & 3)).  Fragments are read with the gfx950
// transposing LDS read.  (It runs at roughly a third of ds_read_b128's byte
// rate, so the layer's backward transposes its operands once and uses the
// K-contiguous path; this form serves the stand-alone gradient entry points.)
template <int R, int KB>
struct ROperand {
  static constexpr int CPR = R / 8;
  static constexpr int RPI = 64 / CPR;
  static constexpr int NI = KB / (4 * RPI);
  int col[NI];     // per lane: global column of its chunk (clamped)
  int krl[NI];     // per lane: k-row within the slab

  __device__ void init(const Operand& o, int r0, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int q = 4 * i + wave;
      const int kr = RPI * q + lane / CPR;
      const int c = (lane % CPR) ^ (4 * (kr & 3));
      int n = r0 + 8 * c;
      if (n > o.rows - 8) n = o.rows - 8;
      col[i] = n;
      krl[i] = kr;
    }
  }
  __device__ void issue(const Operand& o, int k0, int K, Q3L_LDS char* dst,
                        int wave) const {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int q = 4 * i + wave;
      int kq = k0 + RPI * q;                    // uniform first k-row
      if (kq > K - 1) kq = K - 1;
      uint64_t p;
      int64_t ld;
      int st;
      pick(o, kq, p, ld, st);
      const int k = k0 + krl[i];
      const uint32_t off =
          k < K ? (uint32_t)(((int64_t)(k - st) * ld + col[i]) * 2) : kOOB;
      dma16(p, off, uni(lds_addr(dst + 1024 * (4 * i + wave))));
    }
  }
};

typedef short i16x4_t __attribute__((ext_vector_type(4)));
__device__ inline u32x4_t ld_tr2(const Q3L_LDS char* p, int second) {
  const i16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((Q3L_LDS i16x4_t*)(p));
  const i16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((Q3L_LDS i16x4_t*)(p + second));
  const u32x2_t ua = __builtin_bit_cast(u32x2_t, a), ub = __builtin_bit_cast(u32x2_t, b);
  return u32x4_t{ua[0], ua[1], ub[0], ub[1]};
}

__device__ inline u32x4_t ld_lds16(const Q3L_LDS char* p) {
  return *reinterpret_cast<const Q3L_LDS u32x4_t*>(p);
}

// ---- tile order -----------------------------------------------------------
__device__ inline void map_tile(int bid, int nb, int ntm, int ntn, int& tm,
                                int& tn) {
  // Consecutive workgroup ids are dispatched round-robin over the 8 XCDs;
  // renumber so XCD x works on one contiguous range of logical tiles.
  const int xcd = bid & 7, slot = bid >> 3;
  const int per = nb >> 3, rem = nb & 7;
  const int logical = (xcd < rem) ? xcd * (per + 1) + slot
                                  : rem * (per + 1) + (xcd - rem) * per + slot;
  constexpr int GM = 8;
  const int in_group = GM * ntn;
  const int group = logical / in_group;
  const int first = group * GM;
  const int gsz = min(ntm - first, GM);
  const int local = logical - group * in_group;
  tm = first + local % gsz;
  tn = local / gsz;
}

// silu(g) = g * sigmoid(g); v_rcp_f32 (1 ulp) instead of an IEEE division.
__device__ inline float sigmoid_f(float g) { return __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }
__device__ inline float silu_f(float g) { return g * sigmoid_f(g); }

// ---- fragment readers -----------------------------------------------------
// K-contiguous tile [rows][KB]: lane reads row wb + 32*i + lane%32, k-chunk
// 2*kk + lane/32 (swizzled).  Addresses: lane base + per-kk offset + i*32 rows.
template <int TT, int KB>
struct KFrag {
  uint32_t base;
  uint32_t koff[KB / 16];
  __device__ void init(int wb, int lane) {
    const int r = wb + (lane & 31), h = lane >> 5, sw = kswz<KB>(lane & 31);
    base = (uint32_t)r * (2 * KB);
#pragma unroll
    for (int kk = 0; kk < KB / 16; ++kk) koff[kk] = (uint32_t)(((2 * kk + h) ^ sw) << 4);
  }
  __device__ void read(const Q3L_LDS char* t, int kk, u32x4_t f[TT]) const {
#pragma unroll
    for (int i = 0; i < TT; ++i) f[i] = ld_lds16(t + base + koff[kk] + 64 * KB * i);
  }
};
// Row-contiguous tile [KB][R] (row stride 2R bytes), transposed reads: in
// 16-lane group g, lane s points at k-row 8*(g/2) + s/4 (+4 for the second
// read), columns wb + 32*i + 16*(g%2) + 4*(s%4) .. +3 (chunks swizzled by
// 4 * (k-row & 3)).
template <int TT, int R>
struct RFrag {
  uint32_t base[TT];
  __device__ void init(int wb, int lane) {
    const int g = (lane >> 4) & 3, sl = lane & 15;
    const uint32_t rowoff = (uint32_t)(8 * (g >> 1) + (sl >> 2)) * (2 * R) + 8 * (sl & 1);
#pragma unroll
    for (int i = 0; i < TT; ++i) {
      const int chunk = (((wb + 32 * i) >> 3) ^ (4 * (sl >> 2))) | (2 * (g & 1) + ((sl & 3) >> 1));
      base[i] = rowoff + (uint32_t)chunk * 16u;
    }
  }
  __device__ void read(const Q3L_LDS char* t, int kk, u32x4_t f[TT]) const {
#pragma unroll
    for (int i = 0; i < TT; ++i) f[i] = ld_tr2(t + base[i] + kk * 16 * (2 * R), 4 * (2 * R));
  }
};

template <int ROWS, int TT, int KB, bool KC> struct OpSel;
template <int ROWS, int TT, int KB> struct OpSel<ROWS, TT, KB, true> {
  KOperand<ROWS, KB> ld;
  KFrag<TT, KB> fr;
};
template <int ROWS, int TT, int KB> struct OpSel<ROWS, TT, KB, false> {
  ROperand<ROWS, KB> ld;
  RFrag<TT, ROWS> fr;
};

template <int N>
__device__ inline void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// ---- the kernel -----------------------------------------------------------
// NS LDS stages of KB-deep slabs: slab kt+NS-1 is requested while slab kt is
// multiplied, so global latency is hidden behind NS-1 slabs of MFMA work.
template <int BM, int BN, int KB, int NS, bool AK, bool BKC, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(const GemmArgs g) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int ABYTES = BM * KB * 2, BBYTES = BN * KB * 2;
  constexpr int STAGE = ABYTES + BBYTES;
  __shared__ __attribute__((aligned(1024))) char smem[NS * STAGE];
  Q3L_LDS char* lds = (Q3L_LDS char*)smem;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = (int)uni((uint32_t)(tid >> 6));
  const int wm = wave >> 1, wn = wave & 1;
  const int ntm = (g.M + BM - 1) / BM, ntn = (g.N + BN - 1) / BN;
  int tm, tn;
  map_tile(blockIdx.x, gridDim.x, ntm, ntn, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  OpSel<BM, TM, KB, AK> oa;
  OpSel<BN, TN, KB, BKC> ob;
  constexpr int LOADS = decltype(oa.ld)::NI + decltype(ob.ld)::NI;  // per slab
  oa.ld.init(g.a, m0, wave, lane);
  ob.ld.init(g.b, n0, wave, lane);
  oa.fr.init(wm * WM, lane);
  ob.fr.init(wn * WN, lane);

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int nk = (g.K + KB - 1) / KB;
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) {
    if (s < nk) {
      oa.ld.issue(g.a, s * KB, g.K, lds + s * STAGE, wave);
      ob.ld.issue(g.b, s * KB, g.K, lds + s * STAGE + ABYTES, wave);
    }
  }

  int cur = 0;                 // stage holding slab kt
  int nxt = NS - 1;            // stage for slab kt + NS - 1
  for (int kt = 0; kt < nk; ++kt) {
    // Slab kt's loads (this wave's) are done once at most the loads of the
    // NS-2 later slabs are outstanding; the barrier makes all waves' loads
    // visible and guarantees every wave finished reading the stage about to
    // be refilled.
    if (kt + NS - 2 < nk) wait_vmcnt<LOADS * (NS - 2)>();
    else wait_vmcnt<0>();
    __syncthreads();
    if (kt + NS - 1 < nk) {
      Q3L_LDS char* nx = lds + nxt * STAGE;
      oa.ld.issue(g.a, (kt + NS - 1) * KB, g.K, nx, wave);
      ob.ld.issue(g.b, (kt + NS - 1) * KB, g.K, nx + ABYTES, wave);
    }
    const Q3L_LDS char* As = lds + cur * STAGE;
    const Q3L_LDS char* Bs = As + ABYTES;
    // Fragments are double-buffered in registers: the reads for step kk+1
    // are in flight while the matrix cores work on step kk.
    u32x4_t af[2][TM], bfr[2][TN];
    oa.fr.read(As, 0, af[0]);
    ob.fr.read(Bs, 0, bfr[0]);
#pragma unroll
    for (int kk = 0; kk < KB / 16; ++kk) {
      if (kk + 1 < KB / 16) {
        oa.fr.read(As, kk + 1, af[(kk + 1) & 1]);
        ob.fr.read(Bs, kk + 1, bfr[(kk + 1) & 1]);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = mfma32(bfr[kk & 1][j], af[kk & 1][i], acc[i][j]);
    }
    // Instruction order for the slab (scheduling groups): the first step's
    // fragment reads, then each later step's reads spread evenly over the
    // matrix instructions of the step before it.  A K-contiguous fragment is
    // one LDS read, a transposed one two.
    {
      constexpr int NR = (AK ? TM : 2 * TM) + (BKC ? TN : 2 * TN);
      constexpr int NM = TM * TN, PER = NM / NR > 0 ? NM / NR : 1;
      constexpr int RPG = NR / NM > 0 ? NR / NM : 1;   // reads per group
      constexpr int NG = NR / RPG;
      __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
#pragma unroll
      for (int kk = 0; kk + 1 < KB / 16; ++kk) {
#pragma unroll
        for (int r = 0; r < NG; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, RPG, 0);
        }
        if (NM - PER * NG > 0) __builtin_amdgcn_sched_group_barrier(0x008, NM - PER * NG, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
    }

    cur = (cur + 1 == NS) ? 0 : cur + 1;
    nxt = (nxt + 1 == NS) ? 0 : nxt + 1;
  }

  // ---- epilogue: lane holds C[m][n..n+3] for each (i, j, q) ----
  const Epilogue& e = g.epi;
  const int hl = 4 * (lane >> 5);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m = m0 + wm * WM + i * 32 + (lane & 31);
    if (m >= g.M) continue;
    if constexpr (EPI == EPI_SILU_MUL) {
#pragma unroll
      for (int j = 0; j < TN; j += 2) {
        const int fbase = (n0 + wn * WN) / 2 + (j / 2) * 32;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int f = fbase + 8 * q + hl;
          if (f >= e.ffn) continue;
          float gv[4], uv[4], fv[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            gv[r] = acc[i][j][4 * q + r];
            uv[r] = acc[i][j + 1][4 * q + r];
            fv[r] = silu_f(gv[r]) * uv[r];
          }
          bf16_t* F = static_cast<bf16_t*>(e.c) + (int64_t)m * e.ldc + f;
          st8(F, u32x2_t{pack2(fv[0], fv[1]), pack2(fv[2], fv[3])});
          if (e.gu) {
            bf16_t* G = static_cast<bf16_t*>(e.gu) + (int64_t)m * e.ldgu + f;
            st8(G, u32x2_t{pack2(gv[0], gv[1]), pack2(gv[2], gv[3])});
            st8(G + e.ffn, u32x2_t{pack2(uv[0], uv[1]), pack2(uv[2], uv[3])});
          }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + wn * WN + j * 32 + 8 * q + hl;
          if (n >= g.N) continue;
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = acc[i][j][4 * q + r];
          if constexpr (EPI == EPI_STORE) {
            if (e.r) {
              const u32x2_t rr = ld8(static_cast<const bf16_t*>(e.r) +
                                     (int64_t)m * e.ldr + n);
              v[0] += lo_f(rr[0]); v[1] += hi_f(rr[0]);
              v[2] += lo_f(rr[1]); v[3] += hi_f(rr[1]);
            }
            st8(static_cast<bf16_t*>(e.c) + (int64_t)m * e.ldc + n,
                u32x2_t{pack2(v[0], v[1]), pack2(v[2], v[3])});
          } else if constexpr (EPI == EPI_PARTIAL) {
            *reinterpret_cast<f32x4_t*>(e.p32 + (int64_t)m * e.ldp + n) =
                f32x4_t{v[0], v[1], v[2], v[3]};
            if (e.c) {
              const u32x2_t rr = ld8(static_cast<const bf16_t*>(e.r) +
                                     (int64_t)m * e.ldr + n);
              st8(static_cast<bf16_t*>(e.c) + (int64_t)m * e.ldc + n,
                  u32x2_t{pack2(v[0] + lo_f(rr[0]), v[1] + hi_f(rr[0])),
                          pack2(v[2] + lo_f(rr[1]), v[3] + hi_f(rr[1]))});
            }
          } else if constexpr (EPI == EPI_SILU_BWD) {
            const bf16_t* G = static_cast<const bf16_t*>(e.r) + (int64_t)m * e.ldr + n;
            const u32x2_t g2 = ld8(G), u2 = ld8(G + e.ffn);
            const float gg[4] = {lo_f(g2[0]), hi_f(g2[0]), lo_f(g2[1]), hi_f(g2[1])};
            const float uu[4] = {lo_f(u2[0]), hi_f(u2[0]), lo_f(u2[1]), hi_f(u2[1])};
            float dg[4], du[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float sg = sigmoid_f(gg[r]);
              dg[r] = v[r] * uu[r] * sg * (1.0f + gg[r] * (1.0f - sg));
              du[r] = v[r] * gg[r] * sg;
            }
            bf16_t* D = static_cast<bf16_t*>(e.c) + (int64_t)m * e.ldc + n;
            st8(D, u32x2_t{pack2(dg[0], dg[1]), pack2(dg[2], dg[3])});
            st8(D + e.ffn, u32x2_t{pack2(du[0], du[1]), pack2(du[2], du[3])});
          } else if constexpr (EPI == EPI_WGRAD) {
            const bool s1 = e.cnseg > 1 && m >= e.cstart[1];
            const bool s2 = e.cnseg > 2 && m >= e.cstart[2];
            float* cb = s2 ? e.cs[2] : (s1 ? e.cs[1] : e.cs[0]);
            const int cst = s2 ? e.cstart[2] : (s1 ? e.cstart[1] : e.cstart[0]);
            f32x4_t* C = reinterpret_cast<f32x4_t*>(cb + (int64_t)(m - cst) * e.ldc + n);
            f32x4_t nv{v[0], v[1], v[2], v[3]};
            if (e.accumulate) nv += *C;
            *C = nv;
          }
        }
      }
    }
  }
}

template <int BM, int BN, int KB, int NS, bool AK, bool BKC>
hipError_t launch_epi(const GemmArgs& g, hipStream_t s) {
  const int ntm = (g.M + BM - 1) / BM, ntn = (g.N + BN - 1) / BN;
  dim3 grid(ntm * ntn), block(256);
#define Q3L_GK(E) \
  hipLaunchKernelGGL((gemm_kernel<BM, BN, KB, NS, AK, BKC, E>), grid, block, 0, s, g)
  switch (g.epi.kind) {
    case EPI_STORE: Q3L_GK(EPI_STORE); break;
    case EPI_PARTIAL: Q3L_GK(EPI_PARTIAL); break;
    case EPI_SILU_MUL: Q3L_GK(EPI_SILU_MUL); break;
    case EPI_SILU_BWD: Q3L_GK(EPI_SILU_BWD); break;
    case EPI_WGRAD: Q3L_GK(EPI_WGRAD); break;
    default: return hipErrorInvalidValue;
  }
#undef Q3L_GK
  return hipGetLastError();
}

template <int BM, int BN, int KB, int NS>
hipError_t launch_layout(const GemmArgs& g, hipStream_t s) {
  const bool ak = g.a.k_contig, bk = g.b.k_contig;
  if (ak && bk) return launch_epi<BM, BN, KB, NS, true, true>(g, s);
  if (ak && !bk) return launch_epi<BM, BN, KB, NS, true, false>(g, s);
  if (!ak && !bk) return launch_epi<BM, BN, KB, NS, false, false>(g, s);
  return launch_epi<BM, BN, KB, NS, false, true>(g, s);
}

}  // namespace

hipError_t gemm_bf16(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.K <= 0) return hipSuccess;
  // Largest tile that still gives at least one workgroup per CU.
  constexpr int kCUs = 256;
  auto tiles = [&](int bm, int bn) {
    return (int64_t)((g.M + bm - 1) / bm) * ((g.N + bn - 1) / bn);
  };
  if (tiles(256, 256) >= kCUs) return launch_layout<256, 256, 64, 2>(g, s);
  if (tiles(256, 128) >= kCUs) return launch_layout<256, 128, 64, 2>(g, s);
  return launch_layout<128, 128, 64, 2>(g, s);
}

}  // namespace q3l
