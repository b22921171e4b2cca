// Causal GQA attention on the gfx950 matrix cores (walkthrough page, Step 5:
// softmax(Q K^T / sqrt(d_h) + causal mask) V, kv head of q head j = j / G),
// forward and backward, flash-style: the L x L score matrix is never stored.
//
// Forward (one workgroup = 4 wave64s sharing one kv head):
//   each wave owns 32 query rows of one q head; the workgroup covers the
//   G' = min(G, 4) q heads of a kv group (times 4/G' row blocks), so every
//   K/V tile staged in LDS serves 128 (row, head) pairs.  K/V tiles of 64
//   keys are double-buffered in LDS, filled by direct global->LDS loads in
//   their natural [key][d] layout (16-byte chunks permuted per row against
//   bank conflicts); V^T operands come from transposing LDS reads.  Scores
//   are computed transposed, S^T = K Q^T, so that each lane owns one query:
//   the online-softmax statistics (running max m, running sum l, the merge
//   rule of the state-placement page's ring-attention section) are per
//   lane, and the probabilities feed O^T = V^T P^T straight from the
//   accumulators.  Output: O (bf16) and the log-sum-exp per query (fp32).
//
// Backward (P recomputed from the saved log-sum-exp):
//   delta = rowsum(dO * O) per query, by a row-sum kernel that runs first;
//   dK/dV kernel: a workgroup owns 128 keys of one kv head (32 per wave; K
//     and V in LDS) and sweeps every q head of the group and every query
//     tile at or after its keys (Q / dO tiles and their LSE / delta by
//     direct loads, transposed operands by transposing reads); dK^T and
//     dV^T accumulate in registers, so the G-head sum (adjoint of
//     repeat_interleave) needs no atomics.  In the stored-dS form it also
//     writes dS = P (dP - delta) (bf16) to a scratch buffer;
//   dQ: from that dS (dQ^T += K^T dS^T, one product), or, in the
//     recomputing form, by a kernel of the forward's shape that recomputes
//     S and dP per key tile.  Both forms give the same bits.
#include <climits>
#include <type_traits>

#include "common.h"
#include "ops.h"

namespace q3l {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int KT = 64;        // keys per tile
constexpr float kTau = 8.0f;  // rescale threshold (log2 units), see the forward
// The dQ-from-dS kernel: LDS stages and waves per workgroup (measured: 3
// stages beat 2 by 3%, 4 gain nothing; 8 waves beat 4).
constexpr int kDqStages = 3;
constexpr int kDqWaves = 8;

struct FwdP {
  int B, L, h_q, h_kv, G, hb, rb;
  const bf16_t* q; int64_t ldq;
  const bf16_t* k; int64_t ldk;
  const bf16_t* v; int64_t ldv;
  bf16_t* o; int64_t ldo;
  float* lse;
  float scale_log2;
  // backward
  const bf16_t* dout; int64_t lddo;
  bf16_t* dq; bf16_t* dk; bf16_t* dv;
  float* delta;   // written by the row-sum kernel, read by the others
  // stored-dS form: the dS blocks of the causal triangle (bf16), ds_nt
  // blocks per (sequence, q head); null for the recomputing form.
  bf16_t* ds; int64_t ds_nt;
  // block state (forward over the keys [k_lo, k_hi) only; unnormalised)
  int k_lo, k_hi;
  float* m_out; float* l_out; float* acc; int64_t ld_acc;
};

// Pack accumulator values i = 8*half .. 8*half+7 (bf16) into a k-operand.
__device__ inline u32x4_t pack_half(const f32x16_t& s, int half) {
  const int b = 8 * half;
  return u32x4_t{pack2(s[b + 0], s[b + 1]), pack2(s[b + 2], s[b + 3]),
                 pack2(s[b + 4], s[b + 5]), pack2(s[b + 6], s[b + 7])};
}

// 2^x with the bare v_exp_f32: results below 2^-126 (probabilities that
// small) flush to zero instead of taking the library's denormal-scaling path.
__device__ inline float exp2_raw(float x) { return __builtin_amdgcn_exp2f(x); }

// Direct global->LDS load of 4 bytes per lane through a buffer resource
// (lane i's dword lands at LDS byte lds_base + 4 i; offsets past the
// resource's range read zeros), written like the 16-byte form in common.h.
__device__ inline void lds_dma4_r(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :: "v"(voff), "s"(r), "s"(lds_base) : "memory", "m0");
}

// LDS row layout of the K/V/Q/dO tiles: a [rows][d_h] bf16 tile
// stored row-major with its 16-byte chunks permuted per row: chunk c of row
// r sits at slot c ^ swz(r).  The LDS serves 256 bytes (64 banks of 4) per
// cycle: 16 lanes of a 16-byte read, 32 lanes of an 8-byte read.  swz(r)
// depends on r mod 16 only and is chosen so that both read patterns find
// 256 distinct bytes in every cycle:
//  - 16-byte reads of 16 aligned consecutive rows at one chunk: swz is a
//    bijection on each aligned block of 16 rows (two 128-byte rows share
//    a bank line when d_h = 64, so there the even and the odd rows each
//    need distinct slots);
//  - transposing 8-byte reads, 32 lanes = 4 aligned rows x 4 consecutive
//    chunks (an aligned quad): the quads c ^ swz(r) of the 4 rows (of the
//    2 rows that share bank lines, at d_h = 64) are distinct, i.e. swz(r) / 4
//    differs between them.
template <int CPR>
__device__ inline int swz(int r) {
  if constexpr (CPR == 16) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Direct global->LDS loads of a [NR rows][DH] bf16 tile: rows r0 ..
// r0+NR-1 of the sequence starting at token tok0 (zeros at rows >= L),
// columns col0 .. col0+DH-1 of a [T][ld] matrix, into an LDS tile in the
// layout above, shared among the NW waves of the workgroup (1 KB per
// wave-instruction).  Instruction j of wave w covers rows RPI (w + NW j) ..
// +RPI-1; RPI NW is a multiple of 16, so the swizzle of a lane's row, and
// with it the lane's byte offset, is the same for every j: one per-lane
// offset, computed once, plus a uniform j (RPI NW ld 2).  Per tile only a
// buffer resource over the tile's rows is built, ending at row L, so rows
// past the sequence read zeros without a per-lane test.
template <int DH, int NR, int NW>
struct TileLoader {
  static constexpr int RB = 2 * DH, CPR = RB / 16, RPI = 1024 / RB, NI = NR / RPI / NW;
  static_assert(NR % (RPI * NW) == 0, "whole instructions per wave");
  static_assert((RPI * NW) % 16 == 0, "row swizzle independent of the instruction");
  uint32_t voff;
  __device__ void init(int64_t ld, int wave, int lane) {
    const int row = RPI * wave + lane / CPR;
    voff = (uint32_t)(row * ld * 2) + 16u * (uint32_t)((lane % CPR) ^ swz<CPR>(row));
  }
  __device__ void load(const bf16_t* base, int64_t ld, int64_t tok0, int col0, int r0, int L,
                       Q3L_LDS char* dst, int wave) const {
    const __amdgpu_buffer_rsrc_t r = buf_rsrc(
        base + (tok0 + r0) * ld + col0, (uint32_t)(((int64_t)(L - r0) * ld - col0) * 2));
#pragma unroll
    for (int j = 0; j < NI; ++j)
      lds_dma16_r(r, voff, (uint32_t)(j * RPI * NW * ld * 2),
                  uni(lds_addr(dst + 1024 * (wave + NW * j))));
  }
};

// The same loads with the per-lane offsets computed per tile (the forward
// uses this form: holding the offsets costs it more registers than the
// per-tile address arithmetic costs it time).
template <int DH, int NR, int NW>
__device__ inline void load_rows_lds(const bf16_t* base, int64_t ld, int64_t tok0, int col0,
                                     int r0, int L, Q3L_LDS char* dst, int wave, int lane) {
  constexpr int RB = 2 * DH, CPR = RB / 16, RPI = 1024 / RB;
  static_assert(NR % (RPI * NW) == 0, "whole instructions per wave");
#pragma unroll
  for (int j = 0; j < NR / RPI / NW; ++j) {
    const int i = wave + NW * j;
    const int row = RPI * i + lane / CPR;
    const int c = (lane % CPR) ^ swz<CPR>(row);
    const int gr = r0 + row;
    const uint32_t off = gr < L ? (uint32_t)(((tok0 + gr) * ld + col0 + 8 * c) * 2) : kOOB;
    lds_dma16((uint64_t)base, off, 0u, uni(lds_addr(dst + 1024 * i)));
  }
}

// Per-lane LDS byte offsets of the transposing reads that build a
// [32 d][16 k] MFMA operand from a tile stored [k rows][d]: 16-lane group g,
// source lane sl points at row 4 (g / 2) + sl / 4 (+8 for the second read)
// of a 16-row block, columns 32 dt + 16 (g % 2) + 4 (sl % 4) .. +3.
// Output: row part `rowt` (add 16 RB per 16-row block) and per-dt column
// parts for the two reads (the second includes its +8 rows).
template <int DH>
struct TrOffsets {
  static constexpr int RB = 2 * DH, CPR = RB / 16, NDT = DH / 32;
  uint32_t rowt;
  uint32_t col[2][NDT];
  // col[i][dt] with rowt added, for dt = 0.  As 4 dt + tc = 4 dt ^ tc, the
  // chunk slot of column block dt is that of block 0 XOR 4 dt: the byte
  // offset for block dt is cx[i] ^ 64 dt (rowt and the tile base do not
  // touch those bits).
  uint32_t cx[2];
  __device__ void init(int lane) {
    const int g = lane >> 4, sl = lane & 15;
    const int tq = 4 * (g >> 1) + (sl >> 2);
    const int tc = 2 * (g & 1) + ((sl & 3) >> 1);
    rowt = (uint32_t)tq * RB + 8u * (sl & 1);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      col[0][dt] = (uint32_t)(((4 * dt + tc) ^ swz<CPR>(tq)) << 4);
      col[1][dt] = (uint32_t)(((4 * dt + tc) ^ swz<CPR>(tq + 8)) << 4) + 8u * RB;
    }
    cx[0] = rowt + col[0][0];
    cx[1] = rowt + col[1][0];
  }
  // The same operand from per-lane bases tb[i] = tile address + cx[i]
  // (plus a constant `extra`): one XOR per read instead of a held address.
  __device__ static u32x4_t read_x(const uint32_t (&tb)[2], uint32_t extra, int blk, int dt) {
    const uint32_t x = 64u * (uint32_t)dt, o = extra + 16u * RB * (uint32_t)blk;
    const u32x2_t a = ld_tr8((const Q3L_LDS void*)(uintptr_t)((tb[0] ^ x) + o));
    const u32x2_t b = ld_tr8((const Q3L_LDS void*)(uintptr_t)((tb[1] ^ x) + o));
    return u32x4_t{a[0], a[1], b[0], b[1]};
  }
  // Operand for 16-row block `blk`, 32-column block dt of tile t.
  __device__ u32x4_t read(const Q3L_LDS char* t, int blk, int dt) const {
    const Q3L_LDS char* r = t + rowt + 16u * RB * blk;
    const u32x2_t a = ld_tr8(r + col[0][dt]), b = ld_tr8(r + col[1][dt]);
    return u32x4_t{a[0], a[1], b[0], b[1]};
  }
};

// ============================ forward =======================================
// STATE: the block form -- only keys in [k_lo, k_hi) (and s <= t) count,
// and the output is the unnormalised state of the parallelism page's
// ring-attention merge: m = the largest scaled score (natural log), l = sum
// of exp(score - m), acc = sum of exp(score - m) v (fp32); rows with no
// visible key get (-inf, 0, 0).
//
// Each K/V tile t is one iteration of two phases of pinned slots (one
// matrix instruction each, scheduling barriers between slots), so a wave's
// own softmax arithmetic runs while its matrix instructions execute:
//   A: the 16 score products of tile t+1 (S^T = K Q^T), each slot carrying
//      two exponentials and row-sum adds of tile t's probabilities and the
//      K fragment read two slots ahead;
//   B: the 16 products O^T += V^T P^T of tile t, each slot carrying the row
//      maximum (and, at the diagonal or the sequence end, the mask) of two
//      of tile t+1's scores and the V^T fragment read two slots ahead.
// After B the running maximum is moved for tile t+1 (rarely: only when it
// grows by more than kTau), rescaling O and l.
template <int DH, bool STATE>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(const FwdP p) {
  constexpr int NKK = DH / 16;   // k-steps over the head dim
  constexpr int NDT = DH / 32;   // 32-row tiles of d
  constexpr int RB = 2 * DH, CPR = RB / 16;
  constexpr int TB = KT * RB;    // one K or V tile
  constexpr int NSA = 2 * NKK;   // A slots (score products)
  constexpr int NSB = 4 * NDT;   // B slots (P V products)
  __shared__ __attribute__((aligned(1024))) char smem[4 * TB];   // 2 K slots, 2 V slots
  Q3L_LDS char* lds = (Q3L_LDS char*)smem;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = (int)uni((uint32_t)(tid >> 6));
  const int l32 = lane & 31, h = lane >> 5;
  const int ngroups = p.G / p.hb;
  const int b = blockIdx.x / (p.h_kv * ngroups);
  const int rem = blockIdx.x % (p.h_kv * ngroups);
  const int kvh = rem / ngroups, hg = rem % ngroups;
  const int QB = 32 * p.rb;
  const int qtile = gridDim.y - 1 - blockIdx.y;   // longest rows first
  const int q0 = qtile * QB;
  const int head = kvh * p.G + hg * p.hb + (wave % p.hb);
  const int qw0 = q0 + 32 * (wave / p.hb);        // this wave's first row
  const int L = p.L;
  const int64_t tok0 = (int64_t)b * L;

  // K/V tiles needed by the workgroup and by this wave, counted from tile
  // tb (0, or the first tile of the key range in the block form).
  const int qend = min(q0 + QB, L);
  const int wave_last = min(qw0 + 31, L - 1);
  const int kend_g = STATE ? min(qend, p.k_hi) : qend;
  const int kend_w = STATE ? min(wave_last + 1, p.k_hi) : wave_last + 1;
  const int tb = STATE ? p.k_lo / KT : 0;
  const int ntiles = (kend_g + KT - 1) / KT - tb;
  const int my_tiles = qw0 < L ? (kend_w + KT - 1) / KT - tb : 0;
  const int qrow = qw0 + l32;

  // Q fragments (second MFMA operand: lane owns query row qw0 + l32).
  u32x4_t qf[NKK];
  {
    const int qr = min(qrow, L - 1);
    const bf16_t* qp = p.q + (tok0 + qr) * p.ldq + (int64_t)head * DH + 8 * h;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qf[kk] = ld16(qp + 16 * kk);
  }

  f32x16_t oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[dt][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  float m_max = -INFINITY;   // block form: the exact row maximum (log2 units)

  if constexpr (STATE) {
    // No key of the range is visible to any row of the workgroup (uniform).
    if (ntiles <= 0) {
      if (qrow < L) {
        float* ap = p.acc + (tok0 + qrow) * p.ld_acc + (int64_t)head * DH;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            *reinterpret_cast<f32x4_t*>(ap + 32 * dt + 8 * j + 4 * h) = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (h == 0) {
          const int64_t si = ((int64_t)b * p.h_q + head) * L + qrow;
          p.m_out[si] = -INFINITY;
          p.l_out[si] = 0.f;
        }
      }
      return;
    }
  }

  // K and V tiles by direct loads from one per-lane offset fixed across
  // tiles (a scalar buffer resource per tile, ending at the sequence end).
  // Iteration t reads K(t+1) and V(t) and starts loading K(t+2) and V(t+1)
  // into the slots K(t) and V(t-1) left.
  auto kslot = [&](int s) { return lds + s * TB; };
  auto vslot = [&](int s) { return lds + (2 + s) * TB; };
  TileLoader<DH, KT, 4> kld, vld;
  kld.init(p.ldk, wave, lane);
  vld.init(p.ldv, wave, lane);
  auto load_k = [&](int t, int s) {
    kld.load(p.k, p.ldk, tok0, kvh * DH, (tb + t) * KT, L, kslot(s), wave);
  };
  auto load_v = [&](int t, int s) {
    vld.load(p.v, p.ldv, tok0, kvh * DH, (tb + t) * KT, L, vslot(s), wave);
  };
  // K fragment of k-step kk, key block c: row 32 c + l32, chunk 2 kk + h
  // at slot (2 kk + h) ^ swz(l32) = 2 kk ^ (h ^ swz): a per-lane base XOR
  // 32 kk, plus the block and slot offsets (multiples of 1 KiB).  The
  // NKK XORed bases are computed once, so each fragment read is one LDS
  // instruction with the block and slot offsets as immediates.
  const uint32_t kbase =
      lds_addr(lds) + (uint32_t)l32 * RB + ((uint32_t)(h ^ swz<CPR>(l32)) << 4);
  uint32_t kx[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) kx[kk] = kbase ^ (32u * kk);
  // V^T operand reads: the two transposing reads of d block dt come from
  // per-lane bases cx[i] ^ 64 dt (TrOffsets::read_x), also computed once.
  TrOffsets<DH> tro;
  tro.init(lane);
  uint32_t vx[2][NDT];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) vx[i][dt] = (lds_addr(lds) + tro.cx[i]) ^ (64u * dt);

  f32x16_t sc[2][2];          // scores of tiles t (slot t % 2) and t+1
  // Mask of tile kv0: element (c, e) holds key kv0 + 4h + off(c, e) with
  // off = 32 c + 8 (e / 4) + e % 4 (a constant), visible iff off <= hi and
  // off >= lo -- two per-lane limits per tile, one compare per element.
  struct Lim { int lo, hi; };
  auto limits = [&](int kv0) __attribute__((always_inline)) {
    const int base = kv0 + 4 * h;
    int hi = min(qrow, L - 1) - base;
    int lo = 0;
    if constexpr (STATE) {
      hi = min(hi, p.k_hi - 1 - base);
      lo = p.k_lo - base;
    }
    return Lim{lo, hi};
  };
  auto visible = [&](const Lim& lm, int c, int e) __attribute__((always_inline)) {
    const int off = 32 * c + 8 * (e >> 2) + (e & 3);
    if constexpr (STATE) return off <= lm.hi && off >= lm.lo;
    return off <= lm.hi;
  };
  auto edge_tile = [&](int kv0) __attribute__((always_inline)) {
    bool e = (kv0 + KT - 1 > qw0) || (kv0 + KT > L);
    if constexpr (STATE) e = e || kv0 < p.k_lo || kv0 + KT > p.k_hi;
    return e;
  };
  // Exchange of the two key halves' row maxima (a VALU lane swap between
  // the half-waves), scaled to log2 units; then the reference maximum moves
  // (and O, l are rescaled) only when a row's maximum exceeds it by more
  // than kTau: exponents stay <= kTau, the result is exact, and the
  // 64-multiply rescale is usually skipped.
  auto settle_max = [&](float mx) __attribute__((always_inline)) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                    false, false);
    mx = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])) * p.scale_log2;
    if constexpr (STATE) m_max = fmaxf(m_max, mx);
    if (__any(mx > m_run + kTau)) {
      const float m_new = fmaxf(m_run, mx);
      // (Block form: a row with no visible key so far, beside rows that
      // rescale, has m_run = m_new = -inf; its O and l are still zero.)
      const float alpha = (STATE && m_new == -INFINITY) ? 0.f : exp2_raw(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[dt][e] *= alpha;
    }
  };

  load_k(0, 0);
  if (ntiles > 1) load_k(1, 1);
  load_v(0, 0);
  wait_vmcnt<0>();
  stage_barrier();
  // Prologue: scores of tile 0 and their row maximum.
  {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sc[0][c][e] = 0.f;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        sc[0][c] = mfma32(ld_lds16((const Q3L_LDS void*)(uintptr_t)(kx[kk] + 32u * RB * c)),
                          qf[kk], sc[0][c]);
    }
    if (my_tiles > 0) {
      const int kv0 = tb * KT;
      float mx = -INFINITY;
      if (edge_tile(kv0)) {
        const Lim lm = limits(kv0);
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            sc[0][c][e] = visible(lm, c, e) ? sc[0][c][e] : -INFINITY;
            mx = fmaxf(mx, sc[0][c][e]);
          }
      } else {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[0][c][e]);
      }
      settle_max(mx);
    }
  }
  stage_barrier();            // K(0) read by every wave before its slot is refilled

  // Iteration t; the slot parity is a compile-time constant (two iterations
  // per trip), so LDS slot offsets are immediates.
  auto iter = [&](int t, auto par) __attribute__((always_inline)) {
    constexpr int s = decltype(par)::value;
    if (t + 2 < ntiles) load_k(t + 2, s);
    if (t + 1 < ntiles) load_v(t + 1, s ^ 1);
    if (t < my_tiles) {
      f32x16_t (&cur)[2] = sc[s];
      f32x16_t (&nx)[2] = sc[s ^ 1];
      // (Block form: a row that has seen no visible key yet keeps m_run =
      // -inf; its masked scores then give exp2(-inf) = 0, not NaN.)
      const float neg = (STATE && m_run == -INFINITY) ? 0.f : -m_run;
      float rs = 0.f;
      u32x4_t pf[4];
      // ---- A: scores of tile t+1, exponentials of tile t ----
      // The wave runs phase A at raised priority: where the other wave on
      // its SIMD (another workgroup, not in step with it) is in phase B, A's
      // instructions go first (1.8% faster than equal priorities).
      __builtin_amdgcn_s_setprio(1);
      {
        auto kfrag = [&](int j) __attribute__((always_inline)) {
          return ld_lds16((const Q3L_LDS void*)(uintptr_t)(
              kx[j >> 1] + (uint32_t)((s ^ 1) * TB) + 32u * RB * (j & 1)));
        };
        u32x4_t ring[3];
        ring[0] = kfrag(0);
        ring[1] = kfrag(1);
#pragma unroll
        for (int j = 0; j < NSA; ++j) {
          const int c = j & 1, kk = j >> 1;
          if (kk == 0) {
#pragma unroll
            for (int e = 0; e < 16; ++e) nx[c][e] = 0.f;
          }
          nx[c] = mfma32(ring[j % 3], qf[kk], nx[c]);
          if (j + 2 < NSA) ring[(j + 2) % 3] = kfrag(j + 2);
          constexpr int EPS = 32 / NSA;   // exponentials per slot
#pragma unroll
          for (int x = 0; x < EPS; ++x) {
            const int q = EPS * j + x, cc = q >> 4, e = q & 15;
            const float pv = exp2_raw(fmaf(cur[cc][e], p.scale_log2, neg));
            cur[cc][e] = pv;
            rs += pv;
            // Each group of 8 probabilities goes to bf16 (an MFMA operand
            // of phase B) as soon as it is complete.
            if ((q & 7) == 7) pf[q >> 3] = pack_half(cur[cc], (q >> 3) & 1);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      l_run += rs;   // this half-wave's keys; the halves are added at the end
      // ---- B: O^T += V^T P^T of tile t, row maximum of tile t+1 ----
      const bool more = t + 1 < my_tiles;   // tile t+1 is this wave's too
      const int kv1 = (tb + t + 1) * KT;
      float mx = -INFINITY;
      // Tiles that reach the diagonal or the sequence end (one or two per
      // row) redo the maximum with the mask in a pass of their own after the
      // slots: a second, masked copy of the pinned slots costs more
      // registers than a wave has.
      auto phase_b = [&](auto with_max) __attribute__((always_inline)) {
        constexpr bool MAX = decltype(with_max)::value;
        auto vfrag = [&](int j) __attribute__((always_inline)) {
          const uint32_t o = (uint32_t)((2 + s) * TB) + 16u * RB * (uint32_t)(j / NDT);
          const int dt = j % NDT;
          const u32x2_t a = ld_tr8((const Q3L_LDS void*)(uintptr_t)(vx[0][dt] + o));
          const u32x2_t b2 = ld_tr8((const Q3L_LDS void*)(uintptr_t)(vx[1][dt] + o));
          return u32x4_t{a[0], a[1], b2[0], b2[1]};
        };
        u32x4_t ring[3];
        ring[0] = vfrag(0);
        ring[1] = vfrag(1);
#pragma unroll
        for (int j = 0; j < NSB; ++j) {
          const int ks = j / NDT, dt = j % NDT;
          oacc[dt] = mfma32(ring[j % 3], pf[ks], oacc[dt]);
          if (j + 2 < NSB) ring[(j + 2) % 3] = vfrag(j + 2);
          if constexpr (MAX) {
            constexpr int MPS = 32 / NSB;   // maxima per slot
#pragma unroll
            for (int x = 0; x < MPS; ++x) {
              const int q = MPS * j + x;
              mx = fmaxf(mx, nx[q >> 4][q & 15]);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      __builtin_amdgcn_s_setprio(0);
      phase_b(std::true_type{});
      if (more && edge_tile(kv1)) {
        mx = -INFINITY;
        const Lim lm = limits(kv1);
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            nx[c][e] = visible(lm, c, e) ? nx[c][e] : -INFINITY;
            mx = fmaxf(mx, nx[c][e]);
          }
      }
      if (more) settle_max(mx);
    }
    wait_vmcnt<0>();
    stage_barrier();
  };
  for (int t = 0; t < ntiles; t += 2) {
    iter(t, std::integral_constant<int, 0>{});
    if (t + 1 < ntiles) iter(t + 1, std::integral_constant<int, 1>{});
  }

  l_run += __shfl_xor(l_run, 32, 64);
  if (qrow >= L) return;
  if constexpr (STATE) {
    // Rescale to the exact row maximum (m_run may trail it by up to kTau).
    const bool none = m_max == -INFINITY;
    const float a = none ? 0.f : exp2_raw(m_run - m_max);
    float* ap = p.acc + (tok0 + qrow) * p.ld_acc + (int64_t)head * DH;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<f32x4_t*>(ap + 32 * dt + 8 * j + 4 * h) =
            none ? f32x4_t{0.f, 0.f, 0.f, 0.f}
                 : f32x4_t{oacc[dt][4 * j] * a, oacc[dt][4 * j + 1] * a,
                           oacc[dt][4 * j + 2] * a, oacc[dt][4 * j + 3] * a};
    if (h == 0) {
      const int64_t si = ((int64_t)b * p.h_q + head) * L + qrow;
      p.m_out[si] = none ? -INFINITY : m_max * kLn2;
      p.l_out[si] = none ? 0.f : l_run * a;
    }
    return;
  }
  const float inv = 1.0f / l_run;
  bf16_t* op = p.o + (tok0 + qrow) * p.ldo + (int64_t)head * DH;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = 32 * dt + 8 * j + 4 * h;
      st8(op + d, u32x2_t{pack2(oacc[dt][4 * j] * inv, oacc[dt][4 * j + 1] * inv),
                          pack2(oacc[dt][4 * j + 2] * inv, oacc[dt][4 * j + 3] * inv)});
    }
  if (h == 0)
    p.lse[((int64_t)b * p.h_q + head) * L + qrow] = (m_run + log2f(l_run)) * kLn2;
}

// ============================ backward ======================================
// dK, dV for 128 keys of one kv head.  Eight waves: wave w owns keys
// 32 (w % 4) .. +31 and, of every QT-query tile, the 32 query rows
// 32 (w / 4) .. +31, so the two waves sharing a SIMD work on independent
// halves of a tile and hide each other's latencies; their dK/dV partial sums
// are added through LDS at the end.  K and V of the workgroup's keys and
// double-buffered Q / dO tiles sit in LDS in the layout above, filled by
// direct global->LDS loads (no registers, no LDS store instructions); the
// wave's K fragments, the same for every query tile, are also held in
// registers (one LDS read per score instruction instead of two; V's would
// not fit beside them at two waves per SIMD); the transposed operands of
// dV^T += dO^T P^T and dK^T += Q^T dS^T come from transposing LDS reads of
// the same tiles.
//
// DS (the stored-dS form): each wave also writes its 32x32 blocks of dS
// (bf16, as packed for the dK^T instructions) to the dS buffer, for the
// dQ-from-dS kernel below.  A block (query block qb, key block kb; 32 rows
// each, kb <= qb) of sequence b, q head j sits at block index
// (qb (qb + 1) / 2 + kb) B h_q + b h_q + j, 2 KB each: the blocks of one
// (qb, kb) for all sequences and heads are adjacent, so the workgroups of
// the dQ kernel, which walk the key blocks in step, read neighbouring
// memory (15% faster than one region per sequence and head).  Inside a block the lane holding key kl (0..31) and
// half h stores its two 16-byte packs hk = 0, 1 (queries 16 hk + 4 h +
// {0..3, 8..11}) at byte 16 (16 (kl / 4) + 8 hk + 4 h + kl % 4): each store
// instruction fills eight whole 128-byte lines, and the transposing reads
// that the dQ kernel makes of the block (32 lanes = 16 packs, both halves)
// hit 32 distinct 8-byte bank pairs.
template <int DH, bool DS>
__global__ __launch_bounds__(512, 1) void attn_dkdv_kernel(const FwdP p) {
  constexpr int NKK = DH / 16, NDT = DH / 32;
  constexpr int QT = 64, KB = 128;             // queries per tile, keys per workgroup
  constexpr int RB = 2 * DH;                   // bytes per row
  constexpr int CPR = RB / 16;                 // 16-byte chunks per row
  constexpr int KVB = KB * RB, TB = QT * RB;
  __shared__ __attribute__((aligned(1024))) char smem[2 * KVB + 4 * TB];
  __shared__ __attribute__((aligned(16))) float sLD[2][2][QT];   // [stage][lse, delta][q]
  Q3L_LDS char* lds = (Q3L_LDS char*)smem;
  Q3L_LDS char* sK = lds;
  Q3L_LDS char* sV = lds + KVB;
  Q3L_LDS float* ldsLD = (Q3L_LDS float*)&sLD[0][0][0];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = (int)uni((uint32_t)(tid >> 6));
  const int wk = wave & 3, half = wave >> 2;   // key block, query half
  const int l32 = lane & 31, h = lane >> 5;
  const int b = blockIdx.x / p.h_kv, kvh = blockIdx.x % p.h_kv;
  const int kb0 = blockIdx.y * KB;
  const int kw0 = kb0 + 32 * wk;          // first key of this wave
  const int L = p.L;
  const int64_t tok0 = (int64_t)b * L;
  const int mykv = kw0 + l32;

  // Query tiles: for each q head of the group, tiles from the one holding
  // key kb0 to the end of the sequence.
  const int qt_first = kb0 / QT;
  const int nqt = (L + QT - 1) / QT - qt_first;
  const int total = nqt * p.G;
  auto stage = [&](int s) { return lds + 2 * KVB + s * 2 * TB; };   // Q, then dO
  TileLoader<DH, QT, 8> qld, old_;
  qld.init(p.ldq, wave, lane);
  old_.init(p.lddo, wave, lane);
  // Tile (head index hi of the group, query tile qi of the nqt): the tile
  // counters advance incrementally (no division per tile).
  auto load_tile = [&](int hi, int qi, int s) {
    const int head = kvh * p.G + hi;
    const int q0 = (qt_first + qi) * QT;
    qld.load(p.q, p.ldq, tok0, head * DH, q0, L, stage(s), wave);
    old_.load(p.dout, p.lddo, tok0, head * DH, q0, L, stage(s) + TB, wave);
    if (wave < 2) {   // log-sum-exp (wave 0) and row sums (wave 1), 64 floats each
      const float* src = (wave == 0 ? (const float*)p.lse : p.delta) +
                         ((int64_t)b * p.h_q + head) * L + q0;
      lds_dma4_r(buf_rsrc(src, (uint32_t)(L - q0) * 4u), 4u * (uint32_t)lane,
                 uni(lds_addr(ldsLD + (2 * s + wave) * QT)));
    }
  };

  {
    TileLoader<DH, KB, 8> kl, vl;
    kl.init(p.ldk, wave, lane);
    vl.init(p.ldv, wave, lane);
    kl.load(p.k, p.ldk, tok0, kvh * DH, kb0, L, sK, wave);
    vl.load(p.v, p.ldv, tok0, kvh * DH, kb0, L, sV, wave);
  }
  load_tile(0, 0, 0);
  wait_vmcnt<0>();
  stage_barrier();

  // Per-lane LDS addresses of the 16-byte reads: rows 32 half + l32 of a
  // Q/dO tile and rows 32 wk + l32 of K/V all have swizzle swz(l32), so
  // chunk 2kk + h sits at slot 2kk ^ (h ^ swz): byte address base ^ (32 kk).
  const uint32_t swc = (uint32_t)(h ^ swz<CPR>(l32)) << 4;
  const uint32_t kbase = lds_addr(sK) + (uint32_t)(32 * wk + l32) * RB + swc;
  const uint32_t qbase = lds_addr(lds) + 2u * KVB + (uint32_t)(32 * half + l32) * RB + swc;
  // Transposing reads for the dO^T / Q^T operands.
  TrOffsets<DH> tro;
  tro.init(lane);

  f32x16_t dkt[NDT], dvt[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) { dkt[dt][e] = 0.f; dvt[dt][e] = 0.f; }
  // The wave's K fragments are the same for every query tile: read once.
  u32x4_t kfr[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
    kfr[kk] = ld_lds16((const Q3L_LDS void*)(uintptr_t)(kbase ^ (uint32_t)(32 * kk)));

  // Stored-dS form: the lane's byte offset inside a block (see above).
  const uint32_t ds_off = 256u * (uint32_t)(l32 >> 2) + 64u * (uint32_t)h + 16u * (uint32_t)(l32 & 3);

  int hcur = 0, qcur = 0;   // the tile of iteration it
  for (int it = 0; it < total; ++it) {
    const int s = it & 1;
    const int qnx = qcur + 1 == nqt ? 0 : qcur + 1;
    const int hnx = qcur + 1 == nqt ? hcur + 1 : hcur;
    if (it + 1 < total) load_tile(hnx, qnx, s ^ 1);
    const int qh0 = (qt_first + qcur) * QT + 32 * half;   // this wave's first row
    __amdgpu_buffer_rsrc_t rds = buf_rsrc(nullptr, 0);
    if constexpr (DS) {
      // This block's 2 KB (none for rows past the sequence: stores dropped).
      const int head = kvh * p.G + hcur;
      const int64_t qb = qh0 / 32, kb = kw0 / 32;
      const int64_t blk = (qb * (qb + 1) / 2 + kb) * (p.B * p.h_q) + (int64_t)b * p.h_q + head;
      rds = buf_rsrc(p.ds + blk * 1024, qh0 < L ? 2048u : 0u);
    }
    // Skip row blocks entirely before this wave's keys (all masked).
    // One block of 32 queries x 32 keys as a fixed sequence of slots, each
    // one matrix instruction plus a share of the vector work that does not
    // depend on it, pinned by scheduling barriers, so the exponentials and
    // dS overlap the matrix instructions of the same wave:
    //   S = Q K^T (NKK slots), then dP = dO V^T (NKK slots) while P =
    //   exp(S - LSE) is formed; dV^T += dO^T P^T (2 NDT slots) while dS =
    //   P (dP - D) is formed; dK^T += Q^T dS^T (2 NDT slots).
    // Fragments are requested two slots ahead (rings of three).  lane: key
    // mykv; element e holds query row qh0 + 8(e/4) + 4h + e%4 (four
    // consecutive rows per e/4, so LSE and D come in float4s).  Blocks
    // that reach the diagonal or the sequence end mask P between the two
    // phases (one copy of the pinned code; a second copy of it costs more
    // registers than there are).
    auto block = [&](bool edge) __attribute__((always_inline)) {
      const Q3L_LDS char* sQ = stage(s);
      f32x16_t sc, dp;
#pragma unroll
      for (int e = 0; e < 16; ++e) { sc[e] = 0.f; dp[e] = 0.f; }
      uint32_t kb = kbase, qb = qbase + (uint32_t)s * 2u * TB;
      asm volatile("" : "+v"(kb), "+v"(qb));
      auto lds16 = [](uint32_t a) __attribute__((always_inline)) {
        return ld_lds16((const Q3L_LDS void*)(uintptr_t)a);
      };
      // Slot j < NKK: S fragments of k-step j; j >= NKK: dP fragments.
      auto frags = [&](int j, u32x4_t& fa, u32x4_t& fb) __attribute__((always_inline)) {
        const int o = j >= NKK;
        const uint32_t x = (uint32_t)(32 * (j - NKK * o));
        fa = lds16((qb ^ x) + (uint32_t)(TB * o));     // Q or dO
        if (o) fb = lds16((kb ^ x) + (uint32_t)KVB);   // V (K is in kfr)
      };
      const int qr0 = 32 * half + 4 * h;               // row of element 0 in the tile
      constexpr int EP = 16 / NKK;                     // exponentials per dP slot
      f32x4_t l4;
      {
        constexpr int NS = 2 * NKK;
        u32x4_t ra[4], rb[4];
        frags(0, ra[0], rb[0]);
        frags(1, ra[1], rb[1]);
        frags(2, ra[2], rb[2]);
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          if (j < NKK)
            sc = mfma32(ra[j % 4], kfr[j], sc);
          else
            dp = mfma32(ra[j % 4], rb[j % 4], dp);
          if (j + 3 < NS) frags(j + 3, ra[(j + 3) % 4], rb[(j + 3) % 4]);
          if (j >= NKK) {
#pragma unroll
            for (int x = 0; x < EP; ++x) {
              const int e = EP * (j - NKK) + x;
              if ((e & 3) == 0)
                l4 = *reinterpret_cast<const f32x4_t*>(&sLD[s][0][qr0 + 8 * (e >> 2)]) * kLog2e;
              sc[e] = exp2_raw(fmaf(sc[e], p.scale_log2, -l4[e & 3]));
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (edge) {
        // Element e (query qh0 + 4h + r) is kept iff mykv <= q < L and
        // mykv < L, i.e. mlo <= r < mhi.
        const int mlo = mykv - qh0 - 4 * h;
        const int mhi = (mykv < L ? L : INT_MIN / 2) - qh0 - 4 * h;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int r = 8 * (e >> 2) + (e & 3);
          sc[e] = (r < mlo || r >= mhi) ? 0.f : sc[e];
        }
      }
      const u32x4_t pf[2] = {pack_half(sc, 0), pack_half(sc, 1)};
      {
        constexpr int NT = 4 * NDT;      // dV slots, then dK slots
        constexpr int DP = 16 / (2 * NDT);   // dS elements per dV slot
        // Slot j: hk = (j / NDT) % 2, d block j % NDT; dO^T for j < 2 NDT,
        // Q^T after.
        uint32_t tb[2] = {lds_addr(sQ) + 32u * RB * half + tro.cx[0],
                          lds_addr(sQ) + 32u * RB * half + tro.cx[1]};
        asm volatile("" : "+v"(tb[0]), "+v"(tb[1]));
        auto trf = [&](int j) __attribute__((always_inline)) {
          return TrOffsets<DH>::read_x(tb, j < 2 * NDT ? (uint32_t)TB : 0u, (j / NDT) % 2, j % NDT);
        };
        u32x4_t rt[4];
        rt[0] = trf(0);
        rt[1] = trf(1);
        rt[2] = trf(2);
        u32x4_t df[2];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const int hk = (j / NDT) % 2, dt = j % NDT;
          if (j < 2 * NDT)
            dvt[dt] = mfma32(rt[j % 4], pf[hk], dvt[dt]);
          else
            dkt[dt] = mfma32(rt[j % 4], df[hk], dkt[dt]);
          if (j + 3 < NT) rt[(j + 3) % 4] = trf(j + 3);
          if (j < 2 * NDT) {
#pragma unroll
            for (int x = 0; x < DP; ++x) {
              const int e = DP * j + x;
              if ((e & 3) == 0)
                l4 = *reinterpret_cast<const f32x4_t*>(&sLD[s][1][qr0 + 8 * (e >> 2)]);
              dp[e] = sc[e] * (dp[e] - l4[e & 3]);
            }
            if (j == 2 * NDT - 1) {
              df[0] = pack_half(dp, 0);
              df[1] = pack_half(dp, 1);
              if constexpr (DS) {
                buf_st16<kNT>(rds, ds_off, df[0]);
                buf_st16<kNT>(rds, ds_off + 128u, df[1]);
              }
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    // Row blocks entirely before this wave's keys are skipped (all masked).
    if (qh0 + 31 >= kw0 && kw0 < L)
      block((qh0 < kw0 + 31) || (qh0 + 32 > L) || (kw0 + 32 > L));
    wait_vmcnt<0>();      // this wave's part of tile it+1 has landed
    stage_barrier();      // everyone's part; stage s fully read
    hcur = hnx;
    qcur = qnx;
  }

  // Waves 4..7 hand their partial sums to waves 0..3 through LDS (the
  // stages are free now): per wave 2 NDT accumulators of 16 floats per lane.
  float* red = (float*)smem;
  constexpr int PW = 2 * NDT * 16 * 64;        // floats per wave
  if (half == 1) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        red[wk * PW + ((2 * dt) * 16 + e) * 64 + lane] = dkt[dt][e];
        red[wk * PW + ((2 * dt + 1) * 16 + e) * 64 + lane] = dvt[dt][e];
      }
  }
  __syncthreads();
  if (half == 1 || mykv >= L) return;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      dkt[dt][e] += red[wk * PW + ((2 * dt) * 16 + e) * 64 + lane];
      dvt[dt][e] += red[wk * PW + ((2 * dt + 1) * 16 + e) * 64 + lane];
    }
  const float sc = p.scale_log2 / kLog2e;   // 1/sqrt(d_h)
  bf16_t* kp = p.dk + (tok0 + mykv) * p.ldk + (int64_t)kvh * DH;
  bf16_t* vp = p.dv + (tok0 + mykv) * p.ldv + (int64_t)kvh * DH;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = 32 * dt + 8 * j + 4 * h;
      st8(kp + d, u32x2_t{pack2(dkt[dt][4 * j] * sc, dkt[dt][4 * j + 1] * sc),
                          pack2(dkt[dt][4 * j + 2] * sc, dkt[dt][4 * j + 3] * sc)});
      st8(vp + d, u32x2_t{pack2(dvt[dt][4 * j], dvt[dt][4 * j + 1]),
                          pack2(dvt[dt][4 * j + 2], dvt[dt][4 * j + 3])});
    }
}

// dQ for 32 query rows per wave (grid and wave roles as in the forward).
// K/V tiles of KT keys are double-buffered in LDS in the swizzled row layout
// by direct loads; the K^T operand of dQ^T += K^T dS^T comes from
// transposing reads of the same K tile.
template <int DH>
__global__ __launch_bounds__(256, 1) void attn_dq_kernel(const FwdP p) {
  constexpr int NKK = DH / 16, NDT = DH / 32;
  constexpr int RB = 2 * DH, CPR = RB / 16;
  constexpr int TB = KT * RB;                  // one K or V tile
  __shared__ __attribute__((aligned(1024))) char smem[4 * TB];
  Q3L_LDS char* lds = (Q3L_LDS char*)smem;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = (int)uni((uint32_t)(tid >> 6));
  const int l32 = lane & 31, h = lane >> 5;
  const int ngroups = p.G / p.hb;
  const int b = blockIdx.x / (p.h_kv * ngroups);
  const int rem = blockIdx.x % (p.h_kv * ngroups);
  const int kvh = rem / ngroups, hg = rem % ngroups;
  const int QB = 32 * p.rb;
  const int qtile = gridDim.y - 1 - blockIdx.y;
  const int q0 = qtile * QB;
  const int head = kvh * p.G + hg * p.hb + (wave % p.hb);
  const int qw0 = q0 + 32 * (wave / p.hb);
  const int L = p.L;
  const int64_t tok0 = (int64_t)b * L;
  const int qend = min(q0 + QB, L);
  const int ntiles = (qend + KT - 1) / KT;
  const int wave_last = min(qw0 + 31, L - 1);
  const int my_tiles = qw0 < L ? wave_last / KT + 1 : 0;
  const int qrow = qw0 + l32;
  const int qr = min(qrow, L - 1);

  // Q and dO fragments of this wave's rows (second MFMA operand).
  u32x4_t qf[NKK], of[NKK];
  {
    const bf16_t* qp = p.q + (tok0 + qr) * p.ldq + (int64_t)head * DH + 8 * h;
    const bf16_t* op = p.dout + (tok0 + qr) * p.lddo + (int64_t)head * DH + 8 * h;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      qf[kk] = ld16(qp + 16 * kk);
      of[kk] = ld16(op + 16 * kk);
    }
  }
  const int64_t sidx = ((int64_t)b * p.h_q + head) * L + qr;
  const float lse2 = p.lse[sidx] * kLog2e;
  auto stage = [&](int s) { return lds + s * 2 * TB; };   // K, then V
  TileLoader<DH, KT, 4> kld, vld;
  kld.init(p.ldk, wave, lane);
  vld.init(p.ldv, wave, lane);
  auto load_tile = [&](int t, int s) {
    kld.load(p.k, p.ldk, tok0, kvh * DH, t * KT, L, stage(s), wave);
    vld.load(p.v, p.ldv, tok0, kvh * DH, t * KT, L, stage(s) + TB, wave);
  };
  // 16-byte reads of rows 32c + l32, chunk 2kk + h, i.e. slot
  // (2kk + h) ^ swz = 2kk ^ (h ^ swz): byte address kbase ^ (32 kk) (+ the
  // row block, stage and K/V offsets, multiples of 256 bytes).
  const uint32_t kbase =
      lds_addr(lds) + (uint32_t)l32 * RB + ((uint32_t)(h ^ swz<CPR>(l32)) << 4);
  TrOffsets<DH> tro;
  tro.init(lane);

  f32x16_t dqt[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) dqt[dt][e] = 0.f;

  // D = rowsum(dO * O) of this lane's row, from the row-sum kernel (launched
  // before this one); the first K/V tile is requested before it is read.
  load_tile(0, 0);
  const float dlt = p.delta[sidx];

  wait_vmcnt<0>();
  stage_barrier();
  for (int t = 0; t < ntiles; ++t) {
    const int s = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1, s ^ 1);
    if (t < my_tiles) {
      const Q3L_LDS char* sK = stage(s);
      const int kv0 = t * KT;
      f32x16_t sc[2], dp[2];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) { sc[c][e] = 0.f; dp[c][e] = 0.f; }
      // S and dP as four interleaved accumulator chains.  Slot j (k-step
      // j / 4, row block (j / 2) % 2, K for even j, V for odd) runs one
      // matrix instruction and requests the fragment of slot j + 3 (a ring
      // of four), so no matrix instruction waits on a fresh LDS read.  The
      // base address is re-derived per tile (an empty asm hides it from
      // loop-invariant hoisting), so the 4 NKK addresses are not all held
      // in registers.
      {
        uint32_t fb = kbase + (uint32_t)s * 2u * TB;
        asm volatile("" : "+v"(fb));
        auto frag = [&](int j) __attribute__((always_inline)) {
          const uint32_t a = (fb ^ (uint32_t)(32 * (j >> 2))) +
                             (uint32_t)(32 * RB * ((j >> 1) & 1) + TB * (j & 1));
          return ld_lds16((const Q3L_LDS void*)(uintptr_t)a);
        };
        constexpr int NS = 4 * NKK;
        u32x4_t ring[4];
#pragma unroll
        for (int j = 0; j < 3; ++j) ring[j] = frag(j);
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          const int kk = j >> 2, c = (j >> 1) & 1;
          if (j & 1)
            dp[c] = mfma32(ring[j & 3], of[kk], dp[c]);
          else
            sc[c] = mfma32(ring[j & 3], qf[kk], sc[c]);
          if (j + 3 < NS) ring[(j + 3) & 3] = frag(j + 3);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // P in place of S; only tiles that reach the diagonal or the sequence
      // end mask, in a loop of their own after the exponentials.
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) sc[c][e] = exp2_raw(fmaf(sc[c][e], p.scale_log2, -lse2));
      if ((kv0 + KT - 1 > qw0) || (kv0 + KT > L)) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int kv = kv0 + 32 * c + 8 * (e >> 2) + 4 * h + (e & 3);
            sc[c][e] = (kv > qrow || kv >= L) ? 0.f : sc[c][e];
          }
      }
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) dp[c][e] = sc[c][e] * (dp[c][e] - dlt);
      // dQ^T += K^T dS^T: slot j (k-step j / NDT, d block j % NDT) runs one
      // matrix instruction and requests the transposed K fragment of slot
      // j + 2 (a ring of three).
      {
        constexpr int NQ = 4 * NDT;
        u32x4_t ring[3];
        ring[0] = tro.read(sK, 0, 0);
        ring[1] = tro.read(sK, 1 / NDT, 1 % NDT);
        u32x4_t df = pack_half(dp[0], 0);
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
          const int ks = j / NDT, dt = j % NDT;
          if (dt == 0 && j > 0) df = pack_half(dp[ks >> 1], ks & 1);
          dqt[dt] = mfma32(ring[j % 3], df, dqt[dt]);
          if (j + 2 < NQ) ring[(j + 2) % 3] = tro.read(sK, (j + 2) / NDT, (j + 2) % NDT);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    wait_vmcnt<0>();
    stage_barrier();
  }

  if (qrow >= L) return;
  const float sc = p.scale_log2 / kLog2e;
  bf16_t* dp_ = p.dq + (tok0 + qrow) * p.ldq + (int64_t)head * DH;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = 32 * dt + 8 * j + 4 * h;
      st8(dp_ + d, u32x2_t{pack2(dqt[dt][4 * j] * sc, dqt[dt][4 * j + 1] * sc),
                           pack2(dqt[dt][4 * j + 2] * sc, dqt[dt][4 * j + 3] * sc)});
    }
}

// Row sums D = rowsum(dO * O) (fp32) per (sequence, q head, query), read by
// both dQ kernels and by dK/dV.  A workgroup takes 4 passes of 256 / (d_h / 8)
// rows of one q head: each lane loads 16 bytes of dO and of O (a pass reads
// whole rows, contiguous), multiplies in fp32, and the d_h / 8 lanes of a row
// sum their partials by lane exchanges.
template <int DH>
__global__ __launch_bounds__(256) void attn_delta_kernel(const FwdP p) {
  constexpr int LPR = DH / 8;                  // lanes per row
  constexpr int RPP = 256 / LPR;               // rows per pass
  constexpr int NP = 4;                        // passes
  const int t = threadIdx.x, c = t % LPR;
  const int b = blockIdx.x / p.h_q, head = blockIdx.x % p.h_q;
  const int L = p.L;
  const int64_t tok0 = (int64_t)b * L;
  u32x4_t of[NP], ov[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int q = (blockIdx.y * NP + i) * RPP + t / LPR;
    of[i] = ov[i] = u32x4_t{0u, 0u, 0u, 0u};
    if (q < L) {
      of[i] = ld16(p.dout + (tok0 + q) * p.lddo + (int64_t)head * DH + 8 * c);
      ov[i] = ld16(p.o + (tok0 + q) * p.ldo + (int64_t)head * DH + 8 * c);
    }
  }
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    float d = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      d += lo_f(of[i][w]) * lo_f(ov[i][w]) + hi_f(of[i][w]) * hi_f(ov[i][w]);
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) d += __shfl_xor(d, m, 64);
    const int q = (blockIdx.y * NP + i) * RPP + t / LPR;
    if (c == 0 && q < L) p.delta[((int64_t)b * p.h_q + head) * L + q] = d;
  }
}

// dQ from the stored dS: dQ^T += K^T dS^T over the key blocks at or before
// each query block, with no recomputation of S or dP.  A workgroup of NW
// waves shares one kv head; each wave owns 64 query rows (two 32-row query
// blocks) of one q head of the group, so every transposed K fragment read
// from LDS feeds two matrix instructions.  Per tile of 32 keys (one key
// block) the workgroup loads the K tile (shared) and each wave its two dS
// blocks (zeros for a block past the diagonal or the sequence end: its
// products then add nothing), NST stages deep, all by direct global->LDS
// loads; dS, read once, with the non-temporal policy (11% faster: the K
// tiles that other workgroups re-read stay in the L2).  The accumulation
// order is the recomputing dQ kernel's (d block by d block, 16-key steps in
// key order, the same transposed K fragments), so both forms give the same
// bits.  The kernel is bound by its loads (alone they take 197 of its
// 201 us; the products alone 155).  The dS^T operand (lane = query, eight
// keys) comes from transposing reads of a block as the dK/dV kernel stored
// it: for 16-key step ks, source lane sl of 16-lane group g reads keys
// 16 ks + 4 (g / 2) + sl / 4 (+8 for the second read), queries
// 16 (g % 2) + 4 (sl % 4) .. +3, i.e. the 8 bytes at 1024 ks + 256 (g / 2) +
// 128 (g % 2) + 64 (sl % 2) + 16 (sl / 4) + 8 ((sl / 2) % 2) (+512).
template <int DH, int NW, int NST>
__global__ __launch_bounds__(64 * NW, 8 / NW) void attn_dq_ds_kernel(const FwdP p) {
  constexpr int NDT = DH / 32, RB = 2 * DH;
  constexpr int KTS = 32;                      // keys per tile
  constexpr int TB = KTS * RB;                 // one K tile
  constexpr int LW = TB / 1024 < NW ? TB / 1024 : NW;   // waves loading it
  constexpr int KI = TB / 1024 / LW;           // their K load instructions per tile
  constexpr int WB = 4096;                     // a wave's two dS blocks
  constexpr int SB = TB + NW * WB;             // one stage
  __shared__ __attribute__((aligned(1024))) char smem[NST * SB];
  Q3L_LDS char* lds = (Q3L_LDS char*)smem;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = (int)uni((uint32_t)(tid >> 6));
  const int l32 = lane & 31, h = lane >> 5;
  const int ngroups = p.G / p.hb;
  const int b = blockIdx.x / (p.h_kv * ngroups);
  const int rem = blockIdx.x % (p.h_kv * ngroups);
  const int kvh = rem / ngroups, hg = rem % ngroups;
  const int QB = 64 * (NW / p.hb);
  const int qtile = gridDim.y - 1 - blockIdx.y;
  const int q0 = qtile * QB;
  const int head = kvh * p.G + hg * p.hb + (wave % p.hb);
  const int qw0 = q0 + 64 * (wave / p.hb);
  const int L = p.L;
  const int64_t tok0 = (int64_t)b * L;
  const int qend = min(q0 + QB, L);
  const int ntiles = (qend + KTS - 1) / KTS;
  const int my_tiles = qw0 < L ? min(qw0 + 63, L - 1) / KTS + 1 : 0;
  const int64_t qb0 = qw0 / 32;                // this wave's first query block
  const int64_t nbh = (int64_t)p.B * p.h_q;    // blocks between neighbouring key blocks
  const int64_t bh = (int64_t)b * p.h_q + head;
  // dS block (qb, kb) of this (sequence, head).
  auto block = [&](int64_t qb, int64_t kb) {
    return p.ds + ((qb * (qb + 1) / 2 + kb) * nbh + bh) * 1024;
  };

  auto stage = [&](int s) { return lds + s * SB; };
  TileLoader<DH, KTS, LW> kld;
  if (wave < LW) kld.init(p.ldk, wave, lane);
  auto load_tile = [&](int t, int s) {
    if (wave < LW) kld.load(p.k, p.ldk, tok0, kvh * DH, t * KTS, L, stage(s), wave);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bool ok = t < my_tiles && t <= qb0 + c && qw0 + 32 * c < L;
      const __amdgpu_buffer_rsrc_t r = buf_rsrc(ok ? block(qb0 + c, t) : p.ds, ok ? 2048u : 0u);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        lds_dma16_nt(r, 16u * (uint32_t)lane, (uint32_t)(1024 * j),
                     uni(lds_addr(stage(s) + TB + wave * WB + 2048 * c + 1024 * j)));
    }
  };
  TrOffsets<DH> tro;
  tro.init(lane);
  const int g = lane >> 4, sl = lane & 15;
  const uint32_t dsl = 256u * (uint32_t)(g >> 1) + 128u * (uint32_t)(g & 1) +
                       64u * (uint32_t)(sl & 1) + 16u * (uint32_t)(sl >> 2) +
                       8u * (uint32_t)((sl >> 1) & 1);

  f32x16_t dqt[2][NDT];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) dqt[c][dt][e] = 0.f;

#pragma unroll
  for (int i = 0; i < NST - 1; ++i)
    if (i < ntiles) load_tile(i, i);
  for (int t = 0; t < ntiles; ++t) {
    const int s = t % NST;
    // Tile t has landed (later tiles may still be in flight: NST - 2 of
    // them, 4 (+KI) instructions each), then everyone's part of it; the
    // stage read in iteration t - 1 is free for tile t + NST - 1.
    if (t + NST - 2 < ntiles) {
      if (wave < LW) wait_vmcnt<(4 + KI) * (NST - 2)>();
      else wait_vmcnt<4 * (NST - 2)>();
    } else {
      wait_vmcnt<0>();
    }
    stage_barrier();
    if (t + NST - 1 < ntiles) load_tile(t + NST - 1, (t + NST - 1) % NST);
    if (t < my_tiles) {
      const Q3L_LDS char* sK = stage(s);
      const uint32_t db = lds_addr(stage(s) + TB + wave * WB) + dsl;
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        u32x4_t df[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const uint32_t a = db + 2048u * c + 1024u * k2;
          const u32x2_t x0 = ld_tr8((const Q3L_LDS void*)(uintptr_t)a);
          const u32x2_t x1 = ld_tr8((const Q3L_LDS void*)(uintptr_t)(a + 512u));
          df[c] = u32x4_t{x0[0], x0[1], x1[0], x1[1]};
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const u32x4_t kf = tro.read(sK, k2, dt);
          dqt[0][dt] = mfma32(kf, df[0], dqt[0][dt]);
          dqt[1][dt] = mfma32(kf, df[1], dqt[1][dt]);
        }
      }
    }
  }

  const float sc = p.scale_log2 / kLog2e;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int qrow = qw0 + 32 * c + l32;
    if (qrow >= L) continue;
    bf16_t* dp_ = p.dq + (tok0 + qrow) * p.ldq + (int64_t)head * DH;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * dt + 8 * j + 4 * h;
        st8(dp_ + d, u32x2_t{pack2(dqt[c][dt][4 * j] * sc, dqt[c][dt][4 * j + 1] * sc),
                             pack2(dqt[c][dt][4 * j + 2] * sc, dqt[c][dt][4 * j + 3] * sc)});
      }
  }
}

FwdP make_params(const AttnArgs& a) {
  FwdP p{};
  p.B = a.B; p.L = a.L; p.h_q = a.h_q; p.h_kv = a.h_kv;
  p.G = a.h_q / a.h_kv;
  p.hb = (p.G % 4 == 0) ? 4 : (p.G % 2 == 0) ? 2 : 1;
  p.rb = 4 / p.hb;
  p.q = (const bf16_t*)a.q; p.ldq = a.ldq;
  p.k = (const bf16_t*)a.k; p.ldk = a.ldk;
  p.v = (const bf16_t*)a.v; p.ldv = a.ldv;
  p.o = (bf16_t*)a.o; p.ldo = a.ldo;
  p.lse = a.lse;
  p.scale_log2 = kLog2e / sqrtf((float)a.d_h);
  p.dout = (const bf16_t*)a.dout; p.lddo = a.lddo;
  p.dq = (bf16_t*)a.dq; p.dk = (bf16_t*)a.dk; p.dv = (bf16_t*)a.dv;
  p.delta = a.delta;
  p.ds = (bf16_t*)a.ds;
  p.ds_nt = attn_ds_blocks(a.L);
  return p;
}

}  // namespace

hipError_t attn_fwd_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.B <= 0 || a.L <= 0) return hipSuccess;
  const FwdP p = make_params(a);
  const int QB = 32 * p.rb;
  dim3 grid((unsigned)(p.B * p.h_kv * (p.G / p.hb)), (unsigned)cdiv(p.L, QB));
  if (a.d_h == 128)
    hipLaunchKernelGGL((attn_fwd_kernel<128, false>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<64, false>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t attn_block_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.B <= 0 || a.L <= 0) return hipSuccess;
  FwdP p = make_params(a);
  p.k_lo = a.k_lo; p.k_hi = a.k_hi;
  p.m_out = a.m_out; p.l_out = a.l_out; p.acc = a.acc; p.ld_acc = a.ld_acc;
  const int QB = 32 * p.rb;
  dim3 grid((unsigned)(p.B * p.h_kv * (p.G / p.hb)), (unsigned)cdiv(p.L, QB));
  if (a.d_h == 128)
    hipLaunchKernelGGL((attn_fwd_kernel<128, true>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<64, true>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t attn_bwd_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.B <= 0 || a.L <= 0) return hipSuccess;
  const FwdP p = make_params(a);
  dim3 kgrid((unsigned)(p.B * p.h_kv), (unsigned)cdiv(p.L, 128));
  const int QB = 32 * p.rb;
  dim3 qgrid((unsigned)(p.B * p.h_kv * (p.G / p.hb)), (unsigned)cdiv(p.L, QB));
  // The row sums D first (both forms read them).
  if (a.d_h == 128)
    hipLaunchKernelGGL(attn_delta_kernel<128>, dim3((unsigned)(p.B * p.h_q), (unsigned)cdiv(p.L, 64)),
                       dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(attn_delta_kernel<64>, dim3((unsigned)(p.B * p.h_q), (unsigned)cdiv(p.L, 128)),
                       dim3(256), 0, s, p);
  if (p.ds) {
    // Stored dS: dK/dV (which also writes dS), then dQ from dS.
    dim3 dsgrid(qgrid.x, (unsigned)cdiv(p.L, 64 * (kDqWaves / p.hb)));
    if (a.d_h == 128) {
      hipLaunchKernelGGL((attn_dkdv_kernel<128, true>), kgrid, dim3(512), 0, s, p);
      hipLaunchKernelGGL((attn_dq_ds_kernel<128, kDqWaves, kDqStages>), dsgrid,
                         dim3(64 * kDqWaves), 0, s, p);
    } else {
      hipLaunchKernelGGL((attn_dkdv_kernel<64, true>), kgrid, dim3(512), 0, s, p);
      hipLaunchKernelGGL((attn_dq_ds_kernel<64, kDqWaves, kDqStages>), dsgrid,
                         dim3(64 * kDqWaves), 0, s, p);
    }
    return hipGetLastError();
  }
  // Recomputing form: dQ (recomputing S and dP), then dK/dV.
  if (a.d_h == 128) {
    hipLaunchKernelGGL(attn_dq_kernel<128>, qgrid, dim3(256), 0, s, p);
    hipLaunchKernelGGL((attn_dkdv_kernel<128, false>), kgrid, dim3(512), 0, s, p);
  } else {
    hipLaunchKernelGGL(attn_dq_kernel<64>, qgrid, dim3(256), 0, s, p);
    hipLaunchKernelGGL((attn_dkdv_kernel<64, false>), kgrid, dim3(512), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace q3l
