// bf16 GEMM on the gfx950 matrix cores for the seven projections of the
// Qwen3 decoder layer (walkthrough page, Steps 2, 6 and 9) and their
// input/weight gradients.
//
// C[M, N] = sum_k A(m, k) B(n, k), fp32 accumulation.
//
// Design (one workgroup = 4 wave64s = one BM x BN output tile):
//  - K is consumed in slabs of 64.  Each slab of A and B is staged in LDS
//    as [rows][64 + 8] bf16 (the 8-element pad makes the 16-byte fragment
//    reads of 16 consecutive rows hit distinct banks).  Two LDS stages:
//    the next slab's global loads are in flight while the matrix cores work
//    on the current one; one barrier per slab.
//  - Operands whose rows are not K-contiguous in memory (a weight read as
//    [in, out] for an input gradient, activations read along the token axis
//    for a weight gradient) are loaded as 8 rows of 16 bytes and transposed
//    8x8 in registers before the LDS store, so every operand sits in LDS
//    K-contiguous and the inner loop is identical for all layouts.
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

constexpr int BK = 64;
constexpr int LDK = BK + 8;

__device__ inline int seg_of(const int32_t* start, int nseg, int idx) {
  int s = 0;
  if (nseg > 1 && idx >= start[1]) s = 1;
  if (nseg > 2 && idx >= start[2]) s = 2;
  return s;
}

// ---- operand loaders ------------------------------------------------------
// K-contiguous source: each thread moves 16-byte chunks of ROWS/32 rows; the
// chunk column (kc) is fixed per thread, so row addresses are set up once.
template <int ROWS>
struct KLoader {
  static constexpr int NCH = ROWS / 32;
  const bf16_t* rp[NCH];
  u32x4_t reg[NCH];
  int kc, rl;

  __device__ void init(const Operand& o, int r0, int tid) {
    kc = tid & 7;
    rl = tid >> 3;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      int r = r0 + rl + 32 * i;
      int seg, rr;
      if (o.paired) {
        seg = (r >> 5) & 1;
        rr = (r >> 6) * 32 + (r & 31);
        if (rr >= o.rows) rr = o.rows - 1;
        rp[i] = static_cast<const bf16_t*>(o.p[seg]) + (int64_t)rr * o.ld[seg];
      } else {
        rr = r < o.rows ? r : o.rows - 1;
        seg = seg_of(o.start, o.nseg, rr);
        rp[i] = static_cast<const bf16_t*>(o.p[seg]) +
                (int64_t)(rr - o.start[seg]) * o.ld[seg];
      }
    }
  }
  __device__ void load(int k0, int K) {
    const int k = k0 + kc * 8;
#pragma unroll
    for (int i = 0; i < NCH; ++i)
      reg[i] = (k < K) ? ld16(rp[i] + k) : u32x4_t{0u, 0u, 0u, 0u};
  }
  __device__ void store(bf16_t* lds) const {
#pragma unroll
    for (int i = 0; i < NCH; ++i) st16(lds + (rl + 32 * i) * LDK + kc * 8, reg[i]);
  }
};

// Row-contiguous source (element (r, k) at p[(k - start) * ld + r]): each
// active thread owns one 8 (rows) x 8 (k) block, loads it as 8 k-rows of 16
// bytes (consecutive threads read consecutive 16-byte column chunks) and
// transposes it in registers.
template <int ROWS>
struct TLoader {
  u32x4_t reg[8];
  int rb, kb, col;
  bool active;

  __device__ void init(const Operand& o, int r0, int tid) {
    active = tid < ROWS;
    rb = tid % (ROWS / 8);
    kb = tid / (ROWS / 8);
    col = r0 + 8 * rb;
    if (col > o.rows - 8) col = o.rows - 8;
  }
  __device__ void load(const Operand& o, int k0, int K) {
    if (!active) return;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int k = k0 + 8 * kb + r;
      if (k < K) {
        const int s = seg_of(o.start, o.nseg, k);
        reg[r] = ld16(static_cast<const bf16_t*>(o.p[s]) +
                      (int64_t)(k - o.start[s]) * o.ld[s] + col);
      } else {
        reg[r] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  }
  __device__ void store(bf16_t* lds) const {
    if (!active) return;
    u32x4_t t[8];
    transpose8x8(reg, t);
#pragma unroll
    for (int c = 0; c < 8; ++c) st16(lds + (8 * rb + c) * LDK + 8 * kb, t[c]);
  }
};

template <int ROWS, bool KC> struct LoaderSel;
template <int ROWS> struct LoaderSel<ROWS, true> {
  KLoader<ROWS> l;
  __device__ void init(const Operand& o, int r0, int tid) { l.init(o, r0, tid); }
  __device__ void load(const Operand&, int k0, int K) { l.load(k0, K); }
  __device__ void store(bf16_t* lds) const { l.store(lds); }
};
template <int ROWS> struct LoaderSel<ROWS, false> {
  TLoader<ROWS> l;
  __device__ void init(const Operand& o, int r0, int tid) { l.init(o, r0, tid); }
  __device__ void load(const Operand& o, int k0, int K) { l.load(o, k0, K); }
  __device__ void store(bf16_t* lds) const { l.store(lds); }
};

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

__device__ inline float silu_f(float g) { return g / (1.0f + __expf(-g)); }

// ---- the kernel -----------------------------------------------------------
template <int BM, int BN, bool AK, bool BKC, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(const GemmArgs g) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;
  __shared__ __attribute__((aligned(16))) bf16_t lds[2][(BM + BN) * LDK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ntm = (g.M + BM - 1) / BM, ntn = (g.N + BN - 1) / BN;
  int tm, tn;
  map_tile(blockIdx.x, gridDim.x, ntm, ntn, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  LoaderSel<BM, AK> la;
  LoaderSel<BN, BKC> lb;
  la.init(g.a, m0, tid);
  lb.init(g.b, n0, tid);

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int nk = (g.K + BK - 1) / BK;
  la.load(g.a, 0, g.K);
  lb.load(g.b, 0, g.K);
  la.store(lds[0]);
  lb.store(lds[0] + BM * LDK);
  __syncthreads();

  const int arow = wm * WM + (lane & 31), brow = wn * WN + (lane & 31);
  const int kof = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) {
      la.load(g.a, (kt + 1) * BK, g.K);
      lb.load(g.b, (kt + 1) * BK, g.K);
    }
    const bf16_t* As = lds[kt & 1];
    const bf16_t* Bs = As + BM * LDK;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      u32x4_t af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = ld16(As + (arow + i * 32) * LDK + kk * 16 + kof);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = ld16(Bs + (brow + j * 32) * LDK + kk * 16 + kof);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(bfr[j], af[i], acc[i][j]);
    }
    if (more) {
      la.store(lds[(kt + 1) & 1]);
      lb.store(lds[(kt + 1) & 1] + BM * LDK);
    }
    __syncthreads();
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
              const float sg = 1.0f / (1.0f + __expf(-gg[r]));
              dg[r] = v[r] * uu[r] * sg * (1.0f + gg[r] * (1.0f - sg));
              du[r] = v[r] * gg[r] * sg;
            }
            bf16_t* D = static_cast<bf16_t*>(e.c) + (int64_t)m * e.ldc + n;
            st8(D, u32x2_t{pack2(dg[0], dg[1]), pack2(dg[2], dg[3])});
            st8(D + e.ffn, u32x2_t{pack2(du[0], du[1]), pack2(du[2], du[3])});
          } else if constexpr (EPI == EPI_WGRAD) {
            const int s = seg_of(e.cstart, e.cnseg, m);
            f32x4_t* C = reinterpret_cast<f32x4_t*>(
                e.cs[s] + (int64_t)(m - e.cstart[s]) * e.ldc + n);
            f32x4_t nv{v[0], v[1], v[2], v[3]};
            if (e.accumulate) nv += *C;
            *C = nv;
          }
        }
      }
    }
  }
}

template <int BM, int BN, bool AK, bool BKC>
hipError_t launch_epi(const GemmArgs& g, hipStream_t s) {
  const int ntm = (g.M + BM - 1) / BM, ntn = (g.N + BN - 1) / BN;
  dim3 grid(ntm * ntn), block(256);
  switch (g.epi.kind) {
    case EPI_STORE:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, AK, BKC, EPI_STORE>), grid, block, 0, s, g);
      break;
    case EPI_PARTIAL:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, AK, BKC, EPI_PARTIAL>), grid, block, 0, s, g);
      break;
    case EPI_SILU_MUL:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, AK, BKC, EPI_SILU_MUL>), grid, block, 0, s, g);
      break;
    case EPI_SILU_BWD:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, AK, BKC, EPI_SILU_BWD>), grid, block, 0, s, g);
      break;
    case EPI_WGRAD:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, AK, BKC, EPI_WGRAD>), grid, block, 0, s, g);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int BM, int BN>
hipError_t launch_layout(const GemmArgs& g, hipStream_t s) {
  const bool ak = g.a.k_contig, bk = g.b.k_contig;
  if (ak && bk) return launch_epi<BM, BN, true, true>(g, s);
  if (ak && !bk) return launch_epi<BM, BN, true, false>(g, s);
  if (!ak && !bk) return launch_epi<BM, BN, false, false>(g, s);
  return launch_epi<BM, BN, false, true>(g, s);
}

}  // namespace

hipError_t gemm_bf16(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.K <= 0) return hipSuccess;
  // Largest tile that still gives at least one workgroup per CU.
  constexpr int kCUs = 256;
  auto tiles = [&](int bm, int bn) {
    return (int64_t)((g.M + bm - 1) / bm) * ((g.N + bn - 1) / bn);
  };
  if (tiles(256, 256) >= kCUs) return launch_layout<256, 256>(g, s);
  if (tiles(256, 128) >= kCUs) return launch_layout<256, 128>(g, s);
  return launch_layout<128, 128>(g, s);
}

}  // namespace q3l
