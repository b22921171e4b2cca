// bf16 GEMM on the gfx950 matrix cores for the seven projections of the
// Qwen3 decoder layer (walkthrough page, Steps 2, 6 and 9) and their
// input/weight gradients.
//
// C[M, N] = sum_k A(m, k) B(n, k), fp32 accumulation.
//
// Design (one workgroup = one BM x BN output tile; 256 x 256 with 8 wave64s
// for the layer's large GEMMs, 4 wave64s for smaller tiles):
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
//    transposing LDS read (ds_read_b64_tr_b16), at the byte rate of the
//    16-byte reads when its swizzle keeps the banks apart (below).  The
//    layer's input gradients read the weights this way, and the down and
//    gate/up weight gradients their activations (the other operand a
//    transposed copy).
//  - K-contiguous LDS tiles are [rows][KB] with the 16-byte chunks of row r XOR-swizzled
//    by (r >> 1) & 7, so the 16-byte fragment reads of 16 consecutive rows
//    hit 16 distinct bank groups.  Two LDS stages: the next slab streams in
//    while the matrix cores work on the current one; one barrier per slab.
//    Within a slab each k-step is a fixed sequence of slots (a matrix
//    instruction, one fragment read for the next step, a share of the
//    requests), pinned with scheduling barriers.
//  - The waves form a 2 x (NW/2) grid; each owns a (BM/2) x (2 BN/NW)
//    sub-tile of 32x32 accumulators (v_mfma_f32_32x32x16_bf16): 128 x 64 at
//    256 x 256 with 8 waves, two waves per SIMD so one's LDS reads and
//    barrier waits hide behind the other's matrix instructions.  With 8
//    waves only the first 4 issue the direct loads.  The B fragment is
//    passed as the MFMA's first operand so each lane ends up holding four
//    consecutive output columns of one row: epilogue stores are 8 or 16
//    bytes wide.
//  - Workgroup ids are renumbered so each of the 8 XCDs (own L2) receives a
//    contiguous range of tiles, and tiles are walked in groups of 8 tile
//    rows so concurrently running tiles share A and B panels in L2.
//  - Fused epilogues: residual add (Steps 7 and 10), fp32 partial output for
//    a tensor-parallel share, silu(gate) * up over an interleaved gate/up
//    operand (Step 9), the SwiGLU backward, and fp32 (+=) weight gradients.
#include <type_traits>

#include "common.h"
#include "ops.h"

namespace q3l {
namespace {

// Segment holding index idx of an operand (idx uniform): base pointer, ld
// (elements) and start.  Every field is read from the kernel argument through
// readfirstlane before the select, so the compiler keeps the choice between
// register values instead of folding it into an indexed load of the table;
// the fields of unused segments are read too (never selected), so the reads
// are unconditional and shared by every call.
__device__ inline void pick(const Operand& o, int idx, uint64_t& p, int64_t& ld, int& st) {
  const int n = (int)uni((uint32_t)o.nseg);
  const int s1r = (int)uni((uint32_t)o.start[1]), s2r = (int)uni((uint32_t)o.start[2]);
  const int s1 = n > 1 ? s1r : 0x7fffffff;
  const int s2 = n > 2 ? s2r : 0x7fffffff;
  const uint64_t p0 = uni64((uint64_t)o.p[0]);
  const uint64_t p1 = uni64((uint64_t)o.p[1]);
  const uint64_t p2 = uni64((uint64_t)o.p[2]);
  const int64_t l0 = (int64_t)uni64((uint64_t)o.ld[0]);
  const int64_t l1 = (int64_t)uni64((uint64_t)o.ld[1]);
  const int64_t l2 = (int64_t)uni64((uint64_t)o.ld[2]);
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

template <int R, int KB, int NW>
struct KOperand {
  static constexpr int CPRK = KB / 8;
  static constexpr int RPW = 64 / CPRK;
  static constexpr int NI = R / (NW * RPW);  // wave-instructions per thread per slab
  uint32_t voff[NI];   // per lane: byte offset of its chunk at k0 = 0
  // For the last slab: kOOB where the lane's chunk is past K, else 0.  The
  // chunk's swizzle, and so the chunk, is the same for every instruction of
  // the lane (the rows they cover advance by a multiple of 16), so one mask
  // serves all; voff < 2^31, so voff | kOOB is past the buffer's range.
  uint32_t tmask;
  uint64_t base[NI];   // uniform: segment base of the instruction's rows

  __device__ void init(const Operand& o, int r0, int K, int wave, int lane) {
    const int klast = (K - 1) / KB * KB;
    const int rows = (int)uni((uint32_t)o.rows);
    // One branch on the layout (uniform), then straight-line code per
    // instruction.
    auto each = [&](auto paired) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int q = NW * i + wave;
        const int row = RPW * q + lane / CPRK;
        const int c = (lane % CPRK) ^ kswz<KB>(row);
        int gr = r0 + row;
        uint64_t p;
        int64_t ld;
        int st;
        if constexpr (decltype(paired)::value) {
          const int g0 = r0 + RPW * q;        // uniform: first logical row
          const bool up = (g0 >> 5) & 1;
          const uint64_t pg = uni64((uint64_t)o.p[0]), pu = uni64((uint64_t)o.p[1]);
          const int64_t lg = (int64_t)uni64((uint64_t)o.ld[0]);
          const int64_t lu = (int64_t)uni64((uint64_t)o.ld[1]);
          p = up ? pu : pg;
          ld = up ? lu : lg;
          int pr = (gr >> 6) * 32 + (gr & 31);
          if (pr >= rows) pr = rows - 1;
          voff[i] = (uint32_t)((int64_t)pr * ld * 2 + 16 * c);
        } else {
          int g0 = r0 + RPW * q;
          if (g0 > rows - 1) g0 = rows - 1;
          pick(o, g0, p, ld, st);
          if (gr > rows - 1) gr = rows - 1;
          voff[i] = (uint32_t)((int64_t)(gr - st) * ld * 2 + 16 * c);
        }
        if (i == 0) tmask = (klast + 8 * c < K) ? 0u : kOOB;
        base[i] = p;
      }
    };
    if (uni((uint32_t)o.paired))
      each(std::true_type{});
    else
      each(std::false_type{});
  }
  // Wave-instruction i of the slab starting at k0, into LDS stage `dst`
  // (R * KB * 2 bytes); `last` (uniform) selects the offsets that zero-fill
  // chunks past K.  No per-slab address arithmetic: the slab offset rides in
  // the scalar offset.
  __device__ void issue_one(const Operand&, int i, int k0, int, bool last,
                            Q3L_LDS char* dst, int wave) const {
    lds_dma16(base[i], last ? voff[i] | tmask : voff[i], uni(2u * (uint32_t)k0),
          uni(lds_addr(dst + 1024 * (NW * i + wave))));
  }
};

// ---- row-contiguous operand: [KB k][R] in LDS, read transposed -------------
// Element (r, k) at p[(k - start) * ld + r] (a weight read as [in, out], or
// activations read along the token axis).  The tile sits in LDS as in
// memory, [KB][R]: CPR 16-byte chunks per k-row; wave-instruction q fills
// k-rows RPI*q ..; lane l writes k-row RPI*q + l/CPR, slot l%CPR, holding
// global chunk slot ^ rswz(krow).  Fragments are read with the gfx950
// transposing LDS read, two 8-byte reads per fragment, at the byte rate of
// the 16-byte reads (no bank conflicts).  Measured on the Qwen3-8B weight
// gradients with BOTH operands in this form: 0.44-0.51 of the bf16 peak
// against 0.49-0.51 on two transposed copies; with one operand a copy and
// the other in this form, 0.49-0.59 (the o gradient reads both in place,
// the down and gate/up gradients one).
// Chunk permutation of k-row kr of a row-contiguous tile: the transposing
// fragment reads of 32 lanes cover k-rows {0..3, 8..11} (+16 j) at one pair
// of chunks each, and the eight even values 2 ((kr & 3) | (kr & 8) >> 1)
// put those rows' pairs on eight distinct 32-byte bank windows.
__device__ inline int rswz(int kr) { return 2 * ((kr & 3) | ((kr >> 1) & 4)); }

// MS: 0 one segment; 1 several segments along K, each starting at a
// multiple of KB and all of one row stride (a slab lies in one segment);
// 2 several segments in general.
template <int R, int KB, int NW, int MS>
struct ROperand {
  static constexpr int CPR = R / 8;
  static constexpr int RPI = 64 / CPR;
  static constexpr int NI = KB / (NW * RPI);
  int col[NI];        // per lane: global column of its chunk (clamped)
  int krl[NI];        // per lane: k-row within the slab
  // MS 0 and 1: per-lane byte offsets from the slab's first k-row,
  // computed once, and the same for the last slab with kOOB where the k-row
  // is past K; each request then adds only the uniform slab base (for MS 1,
  // of the segment holding the slab).  MS 2 (weights stacked along K at
  // starts that are not multiples of KB, read without a transposed copy)
  // picks the segment per request.
  uint64_t base0;                 // uniform: segment 0 base
  uint64_t vb1, vb2;              // uniform (MS 1): segment bases minus start * ld * 2
  int st1, st2;                   // uniform (MS 1): segment starts (past K if absent)
  int64_t ld0;                    // uniform: row stride (elements)
  uint32_t voff[NI];
  int ktail;                      // klast + the lane's k-row in instruction 0

  __device__ void init(const Operand& o, int r0, int K, int wave, int lane) {
    base0 = uni64((uint64_t)o.p[0]);
    ld0 = (int64_t)uni64((uint64_t)o.ld[0]);
    if constexpr (MS == 1) {
      // Segment s holds k-rows [st_s, st_{s+1}): k-row k of it is at
      // p_s + (k - st_s) ld 2 = vb_s + k ld 2 (modulo 2^64).
      // (Fixed fields, selected after reading: indexing the argument's
      // arrays with a runtime index would copy them to scratch memory.)
      const int n = (int)uni((uint32_t)o.nseg);
      const int s1 = (int)uni((uint32_t)o.start[1]), s2 = (int)uni((uint32_t)o.start[2]);
      const uint64_t p1 = uni64((uint64_t)o.p[1]), p2 = uni64((uint64_t)o.p[2]);
      st1 = n > 1 ? s1 : 0x7fffffff;
      st2 = n > 2 ? s2 : 0x7fffffff;
      vb1 = n > 1 ? p1 - (uint64_t)((int64_t)s1 * ld0 * 2) : base0;
      vb2 = n > 2 ? p2 - (uint64_t)((int64_t)s2 * ld0 * 2) : base0;
    }
    const int klast = (K - 1) / KB * KB;
    ktail = klast + RPI * wave + lane / CPR;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int q = NW * i + wave;
      const int kr = RPI * q + lane / CPR;
      const int c = (lane % CPR) ^ rswz(kr);
      int n = r0 + 8 * c;
      if (n > o.rows - 8) n = o.rows - 8;
      col[i] = n;
      krl[i] = kr;
      voff[i] = (uint32_t)(((int64_t)kr * ld0 + n) * 2);
    }
  }
  // Offset of instruction i in the last slab: kOOB where its k-row (ktail +
  // RPI NW i) is past K.
  __device__ uint32_t tail(int i, int K) const {
    return ktail + RPI * NW * i < K ? voff[i] : kOOB;
  }
  __device__ void issue_one(const Operand& o, int i, int k0, int K, bool last,
                            Q3L_LDS char* dst, int wave) const {
    const uint32_t lds = uni(lds_addr(dst + 1024 * (NW * i + wave)));
    if constexpr (MS == 0) {
      lds_dma16(base0 + (uint64_t)((int64_t)k0 * ld0 * 2), last ? tail(i, K) : voff[i], 0u, lds);
      return;
    }
    if constexpr (MS == 1) {
      // Segment base by masks: written as selects, the choice makes the
      // compiler keep the loader object in scratch memory.
      const uint64_t m1 = 0ull - (uint64_t)(k0 >= st1), m2 = 0ull - (uint64_t)(k0 >= st2);
      const uint64_t vb = base0 + ((vb1 - base0) & m1) + ((vb2 - vb1) & m2);
      // (readfirstlane: the value is uniform, the compiler cannot tell)
      lds_dma16(uni64(vb + (uint64_t)((int64_t)k0 * ld0 * 2)), last ? tail(i, K) : voff[i], 0u,
                lds);
      return;
    }
    const int q = NW * i + wave;
    int kq = k0 + RPI * q;                    // uniform first k-row
    if (kq > K - 1) kq = K - 1;
    uint64_t p;
    int64_t ld;
    int st;
    pick(o, kq, p, ld, st);
    const int k = k0 + krl[i];
    const uint32_t off =
        k < K ? (uint32_t)(((int64_t)(k - st) * ld + col[i]) * 2) : kOOB;
    lds_dma16(p, off, 0u, lds);
  }
};


// ---- tile order -----------------------------------------------------------
__device__ inline void map_tile(int bid, int nb, int ntm, int ntn, int& tm,
                                int& tn) {
  // Each XCD works on one contiguous range of logical tiles.
  const int logical = xcd_contiguous(bid, nb);
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
// Two matrix-instruction shapes are used (see the kernel): 32x32x16 where
// both operands are K-contiguous, 16x16x32 where one is row-contiguous.
// 32x32x16, K-contiguous tile [rows][KB]: lane reads row wb + 32 i + l%32,
// k-chunk 2 kk + l/32 (swizzled); k-steps are 16 deep.
template <int TT, int KB>
struct KFrag32 {
  uint32_t base;
  uint32_t koff[KB / 16];
  __device__ void init(int wb, int lane) {
    const int r = wb + (lane & 31), h = lane >> 5, sw = kswz<KB>(lane & 31);
    base = (uint32_t)r * (2 * KB);
#pragma unroll
    for (int kk = 0; kk < KB / 16; ++kk) koff[kk] = (uint32_t)(((2 * kk + h) ^ sw) << 4);
  }
  __device__ u32x4_t read(const Q3L_LDS char* t, int kk, int i) const {
    return ld_lds16(t + base + koff[kk] + 64 * KB * i);
  }
};
// 16x16x32: lane l holds rows (or columns) 16 i + l%16 of the wave's block i
// and k = 8 (l/16) .. +7 of k-step kk (32 deep).  K-contiguous tile
// [rows][KB]: lane reads row wb + 16 i + l%16, chunk 4 kk + l/16 (swizzled;
// the swizzle of a 16-row block repeats, so it depends on l%16 only).
template <int TT, int KB>
struct KFrag16 {
  uint32_t base;
  uint32_t koff[KB / 32];
  __device__ void init(int wb, int lane) {
    const int r = wb + (lane & 15), g = lane >> 4, sw = kswz<KB>(lane & 15);
    base = (uint32_t)r * (2 * KB);
#pragma unroll
    for (int kk = 0; kk < KB / 32; ++kk) koff[kk] = (uint32_t)(((4 * kk + g) ^ sw) << 4);
  }
  __device__ u32x4_t read(const Q3L_LDS char* t, int kk, int i) const {
    return ld_lds16(t + base + koff[kk] + 32 * KB * i);
  }
};
// Row-contiguous tile [KB][R] (row stride 2R bytes), transposing reads: in
// 16-lane group g, source lane s points at k-row 8 g + s/4 (+4 for the second
// read) of the k-step, columns wb + 16 i + 4 (s%4) .. +3; the transposing
// read hands output lane s the four k values of column wb + 16 i + s.
template <int TT, int R>
struct RFrag {
  uint32_t base[TT];
  __device__ void init(int wb, int lane) {
    const int g = lane >> 4, sl = lane & 15;
    const int kr = 8 * g + (sl >> 2);
    const uint32_t rowoff = (uint32_t)kr * (2 * R) + 8 * (sl & 1);
#pragma unroll
    for (int i = 0; i < TT; ++i) {
      const int chunk = ((wb + 16 * i) >> 3) + ((sl & 3) >> 1);
      base[i] = rowoff + (uint32_t)(chunk ^ rswz(kr)) * 16u;
    }
  }
  __device__ u32x4_t read(const Q3L_LDS char* t, int kk, int i) const {
    return ld_tr_pair(t + base[i] + kk * 32 * (2 * R), 4 * (2 * R));
  }
};

template <int ROWS, int TT, int KB, int NW, bool KC, int MS, int MI> struct OpSel;
template <int ROWS, int TT, int KB, int NW, int MS, int MI>
struct OpSel<ROWS, TT, KB, NW, true, MS, MI> {
  KOperand<ROWS, KB, NW> ld;
  std::conditional_t<MI == 32, KFrag32<TT, KB>, KFrag16<TT, KB>> fr;
};
template <int ROWS, int TT, int KB, int NW, int MS, int MI>
struct OpSel<ROWS, TT, KB, NW, false, MS, MI> {
  static_assert(MI == 16, "row-contiguous operands use the 16x16x32 shape");
  ROperand<ROWS, KB, NW, MS> ld;
  RFrag<TT, ROWS> fr;
};


// ---- the kernel -----------------------------------------------------------
// NS LDS stages of KB-deep slabs: slab kt+NS-1 is requested while slab kt is
// multiplied, so global latency is hidden behind NS-1 slabs of MFMA work.
// BMS: segment mode of a row-contiguous B operand (ROperand's MS).
template <int BM, int BN, int KB, int NS, int NW, bool AK, bool BKC, int EPI, int BMS>
__global__ __launch_bounds__(64 * NW) void gemm_kernel(const GemmArgs g) {
  constexpr int WGN = NW / 2;                  // waves along N (2 along M)
  constexpr int WM = BM / 2, WN = BN / WGN;
  // Matrix-instruction shape.  v_mfma_f32_16x16x32_bf16 sustains more of the
  // peak than v_mfma_f32_32x32x16_bf16 when two waves feed it, but one wave
  // alone keeps it only half busy, so every stall of a SIMD's other wave
  // costs more.  Measured on the layer's GEMMs: 32x32x16 where both operands
  // are K-contiguous (the loader wave stalls at every slab), 16x16x32 where
  // one is read with the transposing loads (the input gradients: 0.53-0.56
  // of the peak against 0.50-0.52).
  constexpr int MI = (AK && BKC) ? 32 : 16;
  constexpr int TM = WM / MI, TN = WN / MI;   // MI x MI accumulator blocks
  using Acc = std::conditional_t<MI == 32, f32x16_t, f32x4_t>;
  constexpr int AEL = MI == 32 ? 16 : 4;      // accumulator elements per lane
  constexpr int ABYTES = BM * KB * 2, BBYTES = BN * KB * 2;
  constexpr int STAGE = ABYTES + BBYTES;
  // The epilogue reuses the LDS: per wave, the fp32 results of one pass
  // (rows padded by 16 bytes).  A wave's rows are staged in two passes, or
  // 32 rows per pass when it holds an odd number of 32-row blocks.
  constexpr int ERS = (BN / (NW / 2)) * 4 + 16;      // staged row, bytes
  constexpr int EPASS = (BM / 64) % 2 == 0 ? 2 : BM / 64;
  constexpr int EREG = (BM / 2 / EPASS) * ERS;        // per wave
  constexpr int SMEM = NS * STAGE > NW * EREG ? NS * STAGE : NW * EREG;
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];
  Q3L_LDS char* lds = (Q3L_LDS char*)smem;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = (int)uni((uint32_t)(tid >> 6));
  const int wm = wave / WGN, wn = wave % WGN;
  const int ntm = (g.M + BM - 1) / BM, ntn = (g.N + BN - 1) / BN;
  int tm, tn;
  map_tile(blockIdx.x, gridDim.x, ntm, ntn, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // With 8 waves only the first 4 (one per SIMD) issue the global->LDS
  // loads: a wave blocks while its load instructions queue at the address
  // unit, and the other wave on the same SIMD keeps the matrix core fed.
  constexpr int NL = NW >= 8 ? NW / 2 : NW;    // waves that issue the loads
  OpSel<BM, TM, KB, NL, AK, 0, MI> oa;
  OpSel<BN, TN, KB, NL, BKC, BMS, MI> ob;
  constexpr int LOADS = decltype(oa.ld)::NI + decltype(ob.ld)::NI;  // per slab
  oa.ld.init(g.a, m0, g.K, wave, lane);
  ob.ld.init(g.b, n0, g.K, wave, lane);
  oa.fr.init(wm * WM, lane);
  ob.fr.init(wn * WN, lane);

  Acc acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < AEL; ++e) acc[i][j][e] = 0.0f;

  constexpr int KS = KB / (MI == 32 ? 16 : 32);   // k-steps per slab
  static_assert(NS >= 2 && (MI == 16 || KS % 2 == 0), "slab pipeline shape");
  // A slab's requests are spread over SP k-steps: with three or more stages
  // over a whole slab's worth of steps, with two (no slack) all at once.
  constexpr int SP = NS >= 3 ? KS : 1;
  constexpr int NIA = decltype(oa.ld)::NI;
  static_assert(LOADS % SP == 0, "requests split evenly over the steps");
  constexpr int NV = LOADS / SP;               // requests per k-step
  constexpr int NF = TM + TN;                  // fragment reads per k-step
  constexpr int NM = TM * TN;                  // matrix instructions per k-step
  static_assert(NF <= NM, "one fragment read per matrix-instruction slot");
  const int nk = (g.K + KB - 1) / KB;
  const int klast = nk - 1;
  // Requests q0 .. q1-1 (of LOADS) of slab kt into stage dst.
  auto issue = [&](int kt, Q3L_LDS char* dst, int q0, int q1) __attribute__((always_inline)) {
    const bool last = kt == klast;
    // Fully unrolled whatever the code size: the loaders' per-lane offset
    // arrays are then indexed by constants and stay in registers.
#pragma clang loop unroll(full)
    for (int q = 0; q < LOADS; ++q) {
      if (q < q0 || q >= q1) continue;
      if (q < NIA)
        oa.ld.issue_one(g.a, q, kt * KB, g.K, last, dst, wave);
      else
        ob.ld.issue_one(g.b, q - NIA, kt * KB, g.K, last, dst + ABYTES, wave);
    }
  };
  // Fragments.  32x32x16: double-buffered (par in use, par ^ 1 filling),
  // read in the order the matrix instructions consume them.  16x16x32 (twice
  // the instructions and fragments per k-step): held once, each replaced by
  // the next step's right after its last matrix instruction (A'[i] after row
  // i, B'[j] after the last row's instruction j).
  constexpr int NBUF = MI == 32 ? 2 : 1;
  u32x4_t af[NBUF][TM], bfr[NBUF][TN];
  // One k-step in a fixed order of NM slots, row-major over the TM x TN
  // accumulators: slot x holds matrix instruction x (B as the first operand,
  // so each lane ends up with four consecutive output columns of one row),
  // then (if rd) the next step's fragment reads due in that slot, then (if
  // ld) the x-th share of request part `part`.  Nothing moves across slots:
  // a request stalled at the address unit delays only what follows it, and
  // the other wave on the SIMD keeps the matrix core busy meanwhile.
  auto step = [&](int par, bool rd, const Q3L_LDS char* As, const Q3L_LDS char* Bs, int kk,
                  bool ld, int kt, Q3L_LDS char* dst, int part) __attribute__((always_inline)) {
#pragma unroll
    for (int x = 0; x < NM; ++x) {
      const int i = x / TN, j = x % TN;
      if constexpr (MI == 32) {
        acc[i][j] = mfma32(bfr[par][j], af[par][i], acc[i][j]);
        if (rd && x < NF) {
          if (x == 0)
            af[par ^ 1][0] = oa.fr.read(As, kk, 0);
          else if (x <= TN)
            bfr[par ^ 1][x - 1] = ob.fr.read(Bs, kk, x - 1);
          else
            af[par ^ 1][x - TN] = oa.fr.read(As, kk, x - TN);
        }
      } else {
        acc[i][j] = mfma16(bfr[0][j], af[0][i], acc[i][j]);
        if (rd) {
          if (j == TN - 1) af[0][i] = oa.fr.read(As, kk, i);
          if (i == TM - 1) bfr[0][j] = ob.fr.read(Bs, kk, j);
        }
      }
      if (ld) issue(kt, dst, part * NV + x * NV / NM, part * NV + (x + 1) * NV / NM);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Slab kt lives in stage kt % NS.  All stages start filling at once.
  if (wave < NL) {
#pragma unroll
    for (int st = 0; st < NS; ++st) issue(min(st, klast), lds + st * STAGE, 0, LOADS);
  }
  wait_vmcnt<LOADS * (NS - 1)>();
  stage_barrier();
  // While the matrix cores work on k-step kk, the reads for step kk+1 are in
  // flight.
#pragma unroll
  for (int i = 0; i < TM; ++i) af[0][i] = oa.fr.read(lds, 0, i);
#pragma unroll
  for (int j = 0; j < TN; ++j) bfr[0][j] = ob.fr.read(lds + ABYTES, 0, j);

  // The stage barrier sits before the LAST k-step of a slab, whose fragments
  // are already in registers: after it the next slab's first fragments are
  // read, and the stage just drained starts receiving slab kt+NS (part 0
  // now, parts 1.. during the next slab's first steps), all hidden behind
  // matrix instructions.  Before the barrier a wave waits for its own part
  // of slab kt+1; NS-2 younger slabs stay in flight.  Requests past the last
  // slab repeat it into stages nothing reads any more (in the first
  // iteration the pending parts repeat slab NS-1 into its own stage: the
  // same bytes).  Loader and non-loader waves run separate copies of the
  // loop, so neither has a branch around the requests.
  auto main_loop = [&](auto loader) __attribute__((always_inline)) {
    constexpr bool LD = decltype(loader)::value;
    int cur = 0;
    int pend = min(NS - 1, klast);
    Q3L_LDS char* pend_dst = lds + (NS - 1) * STAGE;
    for (int kt = 0; kt < nk - 1; ++kt) {
      const int nxt = cur + 1 == NS ? 0 : cur + 1;
      Q3L_LDS char* As = lds + cur * STAGE;
      const Q3L_LDS char* Bs = As + ABYTES;
#pragma unroll
      for (int kk = 0; kk < KS - 1; ++kk)
        step(kk & 1, true, As, Bs, kk + 1, LD && kk + 1 < SP, pend, pend_dst, kk + 1);
      wait_vmcnt<LOADS * (NS - 2)>();
      stage_barrier();
      const Q3L_LDS char* Nx = lds + nxt * STAGE;
      pend = min(kt + NS, klast);
      pend_dst = As;
      step((KS - 1) & 1, true, Nx, Nx + ABYTES, 0, LD, pend, pend_dst, 0);
      cur = nxt;
    }
    const Q3L_LDS char* As = lds + cur * STAGE;
    const Q3L_LDS char* Bs = As + ABYTES;
#pragma unroll
    for (int kk = 0; kk < KS - 1; ++kk) step(kk & 1, true, As, Bs, kk + 1, false, 0, nullptr, 0);
    step((KS - 1) & 1, false, As, Bs, 0, false, 0, nullptr, 0);
  };
  if (wave < NL)
    main_loop(std::true_type{});
  else
    main_loop(std::false_type{});
  // The last requests (repeats of the final slab into idle stages) must
  // land before the workgroup's LDS is released.
  wait_vmcnt<0>();

  // ---- epilogue ----
  // Lane holds C[m][n..n+3] for each (i, j, q) within the wave's WM x WN
  // sub-tile: 32x32x16: m = i*32 + lane%32, n = j*32 + 8q + 4*(lane/32),
  // q < 4; 16x16x32: m = i*16 + lane%16, n = j*16 + 4*(lane/16), q = 0.
  const Epilogue& e = g.epi;
  constexpr int NQ = MI == 32 ? 4 : 1;
  const int hl = MI == 32 ? 4 * (lane >> 5) : 4 * (lane >> 4);
  const int lr = lane & (MI - 1);
  auto quad = [&](int i, int j, int q) __attribute__((always_inline)) {
    if constexpr (MI == 32)
      return f32x4_t{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                     acc[i][j][4 * q + 3]};
    else
      return acc[i][j];
  };
  if constexpr (EPI == EPI_SILU_BWD) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = m0 + wm * WM + i * MI + lr;
      if (m >= g.M) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          const int n = n0 + wn * WN + j * MI + 8 * q + hl;
          if (n >= g.N) continue;
          const f32x4_t cq = quad(i, j, q);
          const bf16_t* G = static_cast<const bf16_t*>(e.r) + (int64_t)m * e.ldr + n;
          const u32x2_t g2 = ld8(G), u2 = ld8(G + e.ffn);
          const float gg[4] = {lo_f(g2[0]), hi_f(g2[0]), lo_f(g2[1]), hi_f(g2[1])};
          const float uu[4] = {lo_f(u2[0]), hi_f(u2[0]), lo_f(u2[1]), hi_f(u2[1])};
          float dg[4], du[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float v = cq[r];
            const float sg = sigmoid_f(gg[r]);
            dg[r] = v * uu[r] * sg * (1.0f + gg[r] * (1.0f - sg));
            du[r] = v * gg[r] * sg;
          }
          bf16_t* D = static_cast<bf16_t*>(e.c) + (int64_t)m * e.ldc + n;
          st8(D, u32x2_t{pack2(dg[0], dg[1]), pack2(dg[2], dg[3])});
          st8(D + e.ffn, u32x2_t{pack2(du[0], du[1]), pack2(du[2], du[3])});
        }
      }
    }
  } else {
    // Results that the next kernels do not read right away leave with
    // non-temporal stores (streamed past the caches' retention): 40 us less
    // per layer step across the plain, partial-sum and weight-gradient
    // epilogues.  The SwiGLU output is the down projection's next operand and
    // keeps ordinary stores (non-temporal there cost that GEMM 4%).
    // Staged through LDS: once every wave is past its last fragment read,
    // each wave writes its fp32 sub-tile one pass (half, or a third) at a
    // time into its own LDS region and reads it back row-major, so every global access covers
    // whole row segments (16 lanes x 16 bytes of one fp32 row, 128 or 64
    // contiguous bytes of bf16) instead of 16 bytes in each of 32 rows.  A
    // wave's LDS accesses execute in order, so a pass may overwrite the
    // region right after the previous pass's reads.
    static_assert((WN == 64 || WN == 128) && TM % EPASS == 0, "epilogue staging shape");
    constexpr int BPP = TM / EPASS;            // MI-row blocks per pass
    constexpr int PR = MI * BPP;               // rows per pass
    constexpr int LPR = WN / 4;                // lanes per staged row (4 floats each)
    constexpr int RPT = 64 / LPR;              // staged rows per read
    constexpr int NT = PR / RPT;               // reads per pass (plain epilogues)
    Q3L_LDS char* reg = lds + wave * EREG;
    const int mw = m0 + wm * WM, nw = n0 + wn * WN;
    // Global accesses go through buffer resources that start at the wave's
    // first row and end at row M (or after the wave's rows): a lane's byte
    // offset is fixed per matrix and advances by a multiple of the row
    // stride per staged row, rows past M fall outside the resource (loads
    // read zeros, stores are dropped), and a lane whose columns lie past N
    // gets an offset past every resource.  No 64-bit address arithmetic per
    // row.  Results that the next kernels do not read right away leave with
    // non-temporal stores (streamed past the caches' retention); the SwiGLU
    // output, the down projection's next operand, keeps ordinary stores.
    // (The resource fields are uniform; uni() lets the compiler keep them in
    // scalar registers instead of looping over lanes.)
    const int vrows = (int)uni((uint32_t)max(0, min(g.M - mw, WM)));   // the wave's rows inside M
    auto rsrc_rows = [&](const void* base, int64_t ld, int esz) __attribute__((always_inline)) {
      const uint64_t b = uni64((uint64_t)(static_cast<const char*>(base) + (int64_t)mw * ld * esz));
      return buf_rsrc(reinterpret_cast<const void*>(b), uni((uint32_t)((int64_t)vrows * ld * esz)));
    };
    // Plain epilogues: in pass p, lane reads staged row RPT t + lane / LPR
    // (t < NT), columns 4 (lane % LPR) .. +3.  The bf16 residual they add is
    // requested for every pass before the first barrier, so the loads
    // overlap one another and the staging instead of each waiting in turn.
    const int cn = 4 * (lane % LPR), nn = nw + cn, rl = lane / LPR;
    const bool colok = nn < g.N;
    auto loff = [&](int64_t ld, int esz) __attribute__((always_inline)) {
      return colok ? (uint32_t)(((int64_t)rl * ld + nn) * esz) : kOOB;
    };
    // Byte offset of staged row (pass, t) relative to the lane's first row.
    auto roff = [&](int pass, int t, int64_t ld, int esz) __attribute__((always_inline)) {
      return (uint32_t)((int64_t)(pass * PR + RPT * t) * ld * esz);
    };
    const void* resid = nullptr;
    if constexpr (EPI == EPI_STORE) resid = e.r;
    if constexpr (EPI == EPI_PARTIAL) resid = e.c ? e.r : nullptr;
    __amdgpu_buffer_rsrc_t rres = buf_rsrc(nullptr, 0), rc = rres, rp = rres;
    uint32_t ores = 0, oc = 0, op = 0;
    if constexpr (EPI == EPI_STORE || EPI == EPI_PARTIAL) {
      if (resid) { rres = rsrc_rows(resid, e.ldr, 2); ores = loff(e.ldr, 2); }
      if (e.c) { rc = rsrc_rows(e.c, e.ldc, 2); oc = loff(e.ldc, 2); }
      if constexpr (EPI == EPI_PARTIAL) { rp = rsrc_rows(e.p32, e.ldp, 4); op = loff(e.ldp, 4); }
    }
    u32x2_t rr[EPASS][NT];
    // Weight-gradient output segments, read once into registers: selecting
    // among fields of the argument block per lane would make the compiler
    // load them from memory for every row.
    const int wg_nseg = (int)uni((uint32_t)e.cnseg);
    const int wg_st1 = (int)uni((uint32_t)e.cstart[1]), wg_st2 = (int)uni((uint32_t)e.cstart[2]);
    const uint64_t wg_c0 = uni64((uint64_t)e.cs[0]), wg_c1 = uni64((uint64_t)e.cs[1]),
                   wg_c2 = uni64((uint64_t)e.cs[2]);
    // Weight gradients: output rows split into up to three segments.  When
    // the wave's rows lie in one of them (no segment starts inside them),
    // one resource over that segment serves every row; otherwise each row
    // picks its segment.
    bool wone = false;
    __amdgpu_buffer_rsrc_t rw = rres;
    uint32_t ow = 0;
    if constexpr (EPI == EPI_WGRAD) {
      const int sg = (wg_nseg > 2 && mw >= wg_st2) ? 2 : (wg_nseg > 1 && mw >= wg_st1) ? 1 : 0;
      const int sst = sg == 2 ? wg_st2 : sg == 1 ? wg_st1 : 0;
      const int snext = (sg == 0 && wg_nseg > 1) ? wg_st1 : (sg == 1 && wg_nseg > 2) ? wg_st2 : INT_MAX;
      wone = mw + vrows <= snext;
      const uint64_t cb = sg == 2 ? wg_c2 : sg == 1 ? wg_c1 : wg_c0;
      const uint64_t b = uni64(cb + (uint64_t)((int64_t)(mw - sst) * e.ldc * 4));
      rw = buf_rsrc(reinterpret_cast<const void*>(b), uni((uint32_t)((int64_t)vrows * e.ldc * 4)));
      ow = loff(e.ldc, 4);
    }
    if constexpr (EPI == EPI_STORE || EPI == EPI_PARTIAL) {
      if (resid) {
#pragma unroll
        for (int pass = 0; pass < EPASS; ++pass)
#pragma unroll
          for (int t = 0; t < NT; ++t)
            rr[pass][t] = buf_ld8(rres, ores + roff(pass, t, e.ldr, 2));
      }
    }
    stage_barrier();
#pragma unroll
    for (int pass = 0; pass < EPASS; ++pass) {
      const int mp = mw + pass * PR;
#pragma unroll
      for (int ii = 0; ii < BPP; ++ii)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int q = 0; q < NQ; ++q)
            *reinterpret_cast<Q3L_LDS f32x4_t*>(reg + (ii * MI + lr) * ERS +
                                                (j * MI + 8 * q + hl) * 4) =
                quad(pass * BPP + ii, j, q);
      if constexpr (EPI == EPI_SILU_MUL) {
        // Staged row: per 64-column block bb, g in columns 64 bb + 0..31
        // and u in 64 bb + 32..63 (the paired operand interleaves 32-column
        // blocks); f column = nw / 2 + 32 bb + c.  Lane: staged row
        // 8 (t / (WN / 64)) + lane / 8, columns 4 (lane % 8) .. +3 of block
        // t % (WN / 64).
        const __amdgpu_buffer_rsrc_t rf = rsrc_rows(e.c, e.ldc, 2);
        const __amdgpu_buffer_rsrc_t rg = rsrc_rows(e.gu, e.gu ? e.ldgu : 0, 2);
#pragma unroll
        for (int t = 0; t < PR * (WN / 64) / 8; ++t) {
          const int bb = t % (WN / 64), row = 8 * (t / (WN / 64)) + (lane >> 3);
          const int c = 4 * (lane & 7);
          const f32x4_t gv =
              *reinterpret_cast<const Q3L_LDS f32x4_t*>(reg + row * ERS + 256 * bb + 4 * c);
          const f32x4_t uv =
              *reinterpret_cast<const Q3L_LDS f32x4_t*>(reg + row * ERS + 256 * bb + 128 + 4 * c);
          const int f = nw / 2 + 32 * bb + c;
          const int r = pass * PR + row;        // row within the wave's rows
          float fv[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) fv[x] = silu_f(gv[x]) * uv[x];
          const bool fok = f < e.ffn;
          buf_st8(rf, fok ? (uint32_t)(((int64_t)r * e.ldc + f) * 2) : kOOB,
                  u32x2_t{pack2(fv[0], fv[1]), pack2(fv[2], fv[3])});
          if (e.gu) {
            const uint32_t og = fok ? (uint32_t)(((int64_t)r * e.ldgu + f) * 2) : kOOB;
            buf_st8(rg, og, u32x2_t{pack2(gv[0], gv[1]), pack2(gv[2], gv[3])});
            buf_st8(rg, og + (uint32_t)(e.ffn * 2), u32x2_t{pack2(uv[0], uv[1]), pack2(uv[2], uv[3])});
          }
        }
      } else {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int row = RPT * t + lane / LPR;
          f32x4_t v = *reinterpret_cast<const Q3L_LDS f32x4_t*>(reg + row * ERS + 4 * cn);
          if constexpr (EPI == EPI_STORE) {
            if (resid) {
              v[0] += lo_f(rr[pass][t][0]); v[1] += hi_f(rr[pass][t][0]);
              v[2] += lo_f(rr[pass][t][1]); v[3] += hi_f(rr[pass][t][1]);
            }
            buf_st8<kNT>(rc, oc + roff(pass, t, e.ldc, 2),
                         u32x2_t{pack2(v[0], v[1]), pack2(v[2], v[3])});
          } else if constexpr (EPI == EPI_PARTIAL) {
            buf_st16<kNT>(rp, op + roff(pass, t, e.ldp, 4), __builtin_bit_cast(u32x4_t, v));
            if (resid) {
              const u32x2_t r2 = rr[pass][t];
              buf_st8<kNT>(rc, oc + roff(pass, t, e.ldc, 2),
                           u32x2_t{pack2(v[0] + lo_f(r2[0]), v[1] + hi_f(r2[0])),
                                   pack2(v[2] + lo_f(r2[1]), v[3] + hi_f(r2[1]))});
            }
          } else if constexpr (EPI == EPI_WGRAD) {
            if (wone) {
              const uint32_t o = ow + roff(pass, t, e.ldc, 4);
              if (e.accumulate) v += __builtin_bit_cast(f32x4_t, buf_ld16(rw, o));
              buf_st16<kNT>(rw, o, __builtin_bit_cast(u32x4_t, v));
              continue;
            }
            const int m = mp + row;
            if (m >= g.M || nn >= g.N) continue;
            const bool s1 = wg_nseg > 1 && m >= wg_st1;
            const bool s2 = wg_nseg > 2 && m >= wg_st2;
            const uint64_t cb = s2 ? wg_c2 : (s1 ? wg_c1 : wg_c0);
            const int cst = s2 ? wg_st2 : (s1 ? wg_st1 : 0);
            Q3L_GLOBAL f32x4_t* C = reinterpret_cast<Q3L_GLOBAL f32x4_t*>(
                cb + ((uint64_t)(m - cst) * e.ldc + nn) * 4);
            if (e.accumulate) v += *C;
            __builtin_nontemporal_store(v, C);
          }
        }
      }
    }
  }
}

template <int BM, int BN, int KB, int NS, int NW, bool AK, bool BKC, int BMS = 0>
hipError_t launch_epi(const GemmArgs& g, hipStream_t s) {
  const int ntm = (g.M + BM - 1) / BM, ntn = (g.N + BN - 1) / BN;
  dim3 grid(ntm * ntn), block(64 * NW);
#define Q3L_GK(E) \
  hipLaunchKernelGGL((gemm_kernel<BM, BN, KB, NS, NW, AK, BKC, E, BMS>), grid, block, 0, s, g)
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

template <int BM, int BN, int KB, int NS, int NW>
hipError_t launch_layout(const GemmArgs& g, hipStream_t s) {
  const bool ak = g.a.k_contig, bk = g.b.k_contig;
  // Several K segments are supported for a row-contiguous B (weights stacked
  // along K in an input-gradient GEMM) only.
  if (!ak && g.a.nseg > 1) return hipErrorInvalidValue;
  if (ak && bk) return launch_epi<BM, BN, KB, NS, NW, true, true>(g, s);
  if (ak && !bk) {
    if (g.b.nseg == 1) return launch_epi<BM, BN, KB, NS, NW, true, false>(g, s);
    bool aligned = true;
    for (int i = 1; i < g.b.nseg; ++i)
      aligned = aligned && g.b.start[i] % KB == 0 && g.b.ld[i] == g.b.ld[0];
    return aligned ? launch_epi<BM, BN, KB, NS, NW, true, false, 1>(g, s)
                   : launch_epi<BM, BN, KB, NS, NW, true, false, 2>(g, s);
  }
  if (!ak && !bk) {
    if (g.b.nseg > 1) return hipErrorInvalidValue;
    return launch_epi<BM, BN, KB, NS, NW, false, false>(g, s);
  }
  // A row-contiguous with B K-contiguous: no caller forms it (the weight
  // gradients take both operands in one form), so it is not instantiated.
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t gemm_bf16(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.K <= 0) return hipSuccess;
  // Largest tile that still gives at least one workgroup per CU.
  constexpr int kCUs = 256;
  auto tiles = [&](int bm, int bn) {
    return (int64_t)((g.M + bm - 1) / bm) * ((g.N + bn - 1) / bn);
  };
  auto rounds = [&](int64_t t) { return (t + kCUs - 1) / kCUs; };
  if (tiles(256, 256) >= kCUs) {
    // Tiles go to the CUs in rounds, and a ragged last round costs a whole
    // one.  A round of 192 x 256 tiles takes about 0.92 of a round of
    // 256 x 256 tiles (measured at 6144 x 4096 x 8192), so the shorter tile
    // wins where it needs as few rounds (there: 2 rounds of 512 tiles
    // against 1.5 of 384).  K-contiguous operands only: the row-contiguous
    // loader assumes a power-of-two tile height.
    if (g.a.k_contig && g.b.k_contig &&
        23 * rounds(tiles(192, 256)) < 25 * rounds(tiles(256, 256)))
      return launch_epi<192, 256, 64, 2, 8, true, true>(g, s);
    return launch_layout<256, 256, 64, 2, 8>(g, s);
  }
  if (tiles(256, 128) >= kCUs) return launch_layout<256, 128, 64, 2, 4>(g, s);
  return launch_layout<128, 128, 64, 2, 4>(g, s);
}

}  // namespace q3l
