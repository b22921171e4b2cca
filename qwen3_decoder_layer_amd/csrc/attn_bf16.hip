// Causal GQA attention on the gfx950 matrix cores (walkthrough page, Step 5:
// softmax(Q K^T / sqrt(d_h) + causal mask) V, kv head of q head j = j / G),
// forward and backward, flash-style: the L x L score matrix is never stored.
//
// Forward (one workgroup = 4 wave64s sharing one kv head):
//   each wave owns 32 query rows of one q head; the workgroup covers the
//   G' = min(G, 4) q heads of a kv group (times 4/G' row blocks), so every
//   K/V tile staged in LDS serves 128 (row, head) pairs.  K/V tiles of 64
//   keys are double-buffered in LDS (V transposed in registers on the way
//   in).  Scores are computed transposed, S^T = K Q^T, so that each lane owns
//   one query: the online-softmax statistics (running max m, running sum l,
//   the merge rule of the state-placement page's ring-attention section) are
//   per lane, and the probabilities feed O^T = V^T P^T straight from the
//   accumulators.  Output: O (bf16) and the log-sum-exp per query (fp32).
//
// Backward (P recomputed from the saved log-sum-exp):
//   delta = rowsum(dO * O) per query;
//   dK/dV kernel: a workgroup owns 128 keys of one kv head (32 per wave,
//     K and V fragments in registers) and sweeps every q head of the group
//     and every query tile at or after its keys; dK^T and dV^T accumulate in
//     registers, so the G-head sum (adjoint of repeat_interleave) needs no
//     atomics;
//   dQ kernel: the forward's shape, accumulating dQ^T over key tiles.
#include "common.h"
#include "ops.h"

namespace q3l {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int KT = 64;        // keys per tile
constexpr float kTau = 8.0f;  // rescale threshold (log2 units), see the forward
constexpr int KTP = KT + 8;   // padded row length of a transposed tile

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
  const float* delta;
};

__device__ inline u32x4_t zero4() { return u32x4_t{0u, 0u, 0u, 0u}; }

// Two 8-byte LDS reads forming one MFMA k-operand whose 16 k-values, for lane
// group h = lane / 32, are {4h..4h+3} and {8+4h..8+4h+3} of a 16-block (the
// order in which a 32x32 accumulator holds rows).
__device__ inline u32x4_t ld_pair8(const bf16_t* p) {
  const u32x2_t a = ld8(p), b = ld8(p + 8);
  return u32x4_t{a[0], a[1], b[0], b[1]};
}

// Pack accumulator values i = 8*half .. 8*half+7 (bf16) into a k-operand.
__device__ inline u32x4_t pack_half(const f32x16_t& s, int half) {
  const int b = 8 * half;
  return u32x4_t{pack2(s[b + 0], s[b + 1]), pack2(s[b + 2], s[b + 3]),
                 pack2(s[b + 4], s[b + 5]), pack2(s[b + 6], s[b + 7])};
}

// ============================ forward =======================================
template <int DH>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(const FwdP p) {
  constexpr int DHP = DH + 8;
  constexpr int NKK = DH / 16;   // k-steps over the head dim
  constexpr int NDT = DH / 32;   // 32-row tiles of d
  __shared__ __attribute__((aligned(16))) bf16_t sK[2][KT * DHP];
  __shared__ __attribute__((aligned(16))) bf16_t sVt[2][DH * KTP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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

  // K/V tiles needed by the workgroup and by this wave.
  const int qend = min(q0 + QB, L);
  const int ntiles = (qend + KT - 1) / KT;
  const int wave_last = min(qw0 + 31, L - 1);
  const int my_tiles = qw0 < L ? wave_last / KT + 1 : 0;

  // Q fragments (second MFMA operand: lane owns query row qw0 + l32).
  u32x4_t qf[NKK];
  {
    const int qr = min(qw0 + l32, L - 1);
    const bf16_t* qp = p.q + (tok0 + qr) * p.ldq + (int64_t)head * DH + 8 * h;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qf[kk] = ld16(qp + 16 * kk);
  }

  // ---- tile loaders ----
  constexpr int KCH = KT * DH / 8 / 256;  // 16-byte K chunks per thread
  u32x4_t kreg[KCH];
  u32x4_t vreg[8];
  // V^T blocks: key-block index fastest over lanes (conflict-free LDS stores).
  const bool vact = tid < (KT / 8) * (DH / 8);
  const int vkb = tid % (KT / 8), vdb = tid / (KT / 8);
  auto load_tile = [&](int t) {
    const int kv0 = t * KT;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + 256 * i;
      const int row = c / (DH / 8), cc = c % (DH / 8);
      const int kv = kv0 + row;
      kreg[i] = kv < L ? ld16(p.k + (tok0 + kv) * p.ldk + (int64_t)kvh * DH + 8 * cc)
                       : zero4();
    }
    if (vact) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int kv = kv0 + 8 * vkb + r;
        vreg[r] = kv < L ? ld16(p.v + (tok0 + kv) * p.ldv + (int64_t)kvh * DH + 8 * vdb)
                         : zero4();
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + 256 * i;
      const int row = c / (DH / 8), cc = c % (DH / 8);
      st16(&sK[buf][row * DHP + 8 * cc], kreg[i]);
    }
    if (vact) {
      u32x4_t tr[8];
      transpose8x8(vreg, tr);
#pragma unroll
      for (int c = 0; c < 8; ++c) st16(&sVt[buf][(8 * vdb + c) * KTP + 8 * vkb], tr[c]);
    }
  };

  f32x16_t oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[dt][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const int qrow = qw0 + l32;

  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const bool more = t + 1 < ntiles;
    if (more) load_tile(t + 1);
    if (t < my_tiles) {
      const bf16_t* Ks = sK[t & 1];
      const bf16_t* Vt = sVt[t & 1];
      const int kv0 = t * KT;
      f32x16_t s[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int e = 0; e < 16; ++e) s[c][e] = 0.f;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
          s[c] = mfma32(ld16(Ks + (32 * c + l32) * DHP + 16 * kk + 8 * h), qf[kk], s[c]);
      }
      const bool need_mask = (kv0 + KT - 1 > qw0) || (kv0 + KT > L);
      float mx = -INFINITY;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float v = s[c][e];
          if (need_mask) {
            const int kv = kv0 + 32 * c + 8 * (e >> 2) + 4 * h + (e & 3);
            if (kv > qrow || kv >= L) v = -INFINITY;
          }
          s[c][e] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * p.scale_log2;   // log2 units
      // The reference maximum m_run moves (and O, l are rescaled) only when a
      // row's maximum exceeds it by more than kTau: exponents stay <= kTau,
      // the result is exact, and the 64-multiply rescale is usually skipped.
      if (__any(mx > m_run + kTau)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = exp2f(m_run - m_new);
        l_run *= alpha;
        m_run = m_new;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[dt][e] *= alpha;
      }
      const float neg = -m_run;
      float rs = 0.f;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float pv = exp2f(fmaf(s[c][e], p.scale_log2, neg));
          s[c][e] = pv;
          rs += pv;
        }
      rs += __shfl_xor(rs, 32, 64);
      l_run += rs;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4_t pf = pack_half(s[ks >> 1], ks & 1);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          oacc[dt] = mfma32(ld_pair8(Vt + (32 * dt + l32) * KTP + 16 * ks + 4 * h), pf,
                            oacc[dt]);
      }
    }
    if (more) store_tile((t + 1) & 1);
    __syncthreads();
  }

  if (qrow >= L) return;
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
// delta[b, h, t] = sum_d dO[t, h, d] * O[t, h, d]
template <int DH>
__global__ __launch_bounds__(256) void attn_delta_kernel(const FwdP p, float* delta) {
  constexpr int LP = DH / 8;
  const int64_t item = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LP;
  const int j = threadIdx.x % LP;
  const int64_t total = (int64_t)p.B * p.L * p.h_q;
  const bool valid = item < total;
  const int64_t it = valid ? item : 0;
  const int64_t tok = it / p.h_q;
  const int head = (int)(it % p.h_q);
  const u32x4_t a = ld16(p.dout + tok * p.lddo + (int64_t)head * DH + 8 * j);
  const u32x4_t o = ld16(p.o + tok * p.ldo + (int64_t)head * DH + 8 * j);
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) s += lo_f(a[e]) * lo_f(o[e]) + hi_f(a[e]) * hi_f(o[e]);
  s = group_sum(s, LP);
  if (valid && j == 0) {
    const int64_t b = tok / p.L, t = tok % p.L;
    delta[(b * p.h_q + head) * p.L + t] = s;
  }
}

// dK, dV for 128 keys of one kv head.
template <int DH>
__global__ __launch_bounds__(256, 1) void attn_dkdv_kernel(const FwdP p) {
  constexpr int DHP = DH + 8;
  constexpr int NKK = DH / 16, NDT = DH / 32;
  constexpr int QT = 64;   // queries per tile
  // Per stage: Q [QT][DHP], Q^T [DH][QT+8], dO [QT][DHP], dO^T [DH][QT+8].
  constexpr int STAGE = 2 * QT * DHP + 2 * DH * (QT + 8);
  __shared__ __attribute__((aligned(16))) bf16_t smem[2][STAGE];
  __shared__ __attribute__((aligned(16))) float sL[2][QT];
  __shared__ __attribute__((aligned(16))) float sD[2][QT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int b = blockIdx.x / p.h_kv, kvh = blockIdx.x % p.h_kv;
  const int kb0 = blockIdx.y * 128;       // first key of the workgroup
  const int kw0 = kb0 + 32 * wave;        // first key of this wave
  const int L = p.L;
  const int64_t tok0 = (int64_t)b * L;
  const int mykv = kw0 + l32;

  // K and V fragments of this wave's 32 keys (second MFMA operand).
  u32x4_t kf[NKK], vf[NKK];
  {
    const int kr = min(mykv, L - 1);
    const bf16_t* kp = p.k + (tok0 + kr) * p.ldk + (int64_t)kvh * DH + 8 * h;
    const bf16_t* vp = p.v + (tok0 + kr) * p.ldv + (int64_t)kvh * DH + 8 * h;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      kf[kk] = ld16(kp + 16 * kk);
      vf[kk] = ld16(vp + 16 * kk);
    }
  }
  f32x16_t dkt[NDT], dvt[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) { dkt[dt][e] = 0.f; dvt[dt][e] = 0.f; }

  // Query tiles: for each q head of the group, tiles from the one holding
  // key kb0 to the end of the sequence.
  const int qt_first = kb0 / QT;
  const int nqt = (L + QT - 1) / QT - qt_first;
  const int total = nqt * p.G;

  // Loader: threads 0..127 own one 8x8 block of Q, 128..255 one of dO.
  const int sel = tid >> 7, bt = tid & 127;
  const int qb = bt % (QT / 8), db = bt / (QT / 8);
  const bool lact = db < DH / 8;
  u32x4_t reg[8];
  float lreg = 0.f;
  auto load_tile = [&](int it) {
    const int head = kvh * p.G + it / nqt;
    const int q0 = (qt_first + it % nqt) * QT;
    if (lact) {
      const bf16_t* base = sel ? p.dout : p.q;
      const int64_t ld = sel ? p.lddo : p.ldq;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int q = q0 + 8 * qb + r;
        reg[r] = q < L ? ld16(base + (tok0 + q) * ld + (int64_t)head * DH + 8 * db) : zero4();
      }
    }
    if (tid < 2 * QT) {
      const int q = q0 + (tid % QT);
      const int64_t idx = ((int64_t)b * p.h_q + head) * L + min(q, L - 1);
      lreg = tid < QT ? p.lse[idx] * kLog2e : p.delta[idx];
    }
  };
  auto store_tile = [&](int buf) {
    bf16_t* S = smem[buf];
    bf16_t* nat = S + sel * (QT * DHP + DH * (QT + 8));
    bf16_t* tr = nat + QT * DHP;
    if (lact) {
#pragma unroll
      for (int r = 0; r < 8; ++r) st16(nat + (8 * qb + r) * DHP + 8 * db, reg[r]);
      u32x4_t t8[8];
      transpose8x8(reg, t8);
#pragma unroll
      for (int c = 0; c < 8; ++c) st16(tr + (8 * db + c) * (QT + 8) + 8 * qb, t8[c]);
    }
    if (tid < QT) sL[buf][tid] = lreg;
    else if (tid < 2 * QT) sD[buf][tid - QT] = lreg;
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int it = 0; it < total; ++it) {
    const bool more = it + 1 < total;
    if (more) load_tile(it + 1);
    const int q0 = (qt_first + it % nqt) * QT;
    const int buf = it & 1;
    // Skip tiles entirely before this wave's keys (all masked).
    if (q0 + QT - 1 >= kw0 && kw0 < L) {
      const bf16_t* sQ = smem[buf];
      const bf16_t* sQt = sQ + QT * DHP;
      const bf16_t* sO = sQt + DH * (QT + 8);
      const bf16_t* sOt = sO + QT * DHP;
      f32x16_t s[2], dp[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int e = 0; e < 16; ++e) { s[c][e] = 0.f; dp[c][e] = 0.f; }
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const int off = (32 * c + l32) * DHP + 16 * kk + 8 * h;
          s[c] = mfma32(ld16(sQ + off), kf[kk], s[c]);
          dp[c] = mfma32(ld16(sO + off), vf[kk], dp[c]);
        }
      }
      // lane: key mykv; rows q = q0 + 32c + 8(e/4) + 4h + e%4 -- four
      // consecutive rows per (c, e/4), so LSE and delta come in float4s.
      const bool need_mask = (q0 < kw0 + 31) || (q0 + QT > L) || (kw0 + 32 > L);
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int qb = 32 * c + 8 * e4 + 4 * h;
          const f32x4_t lq = *reinterpret_cast<const f32x4_t*>(&sL[buf][qb]);
          const f32x4_t dq4 = *reinterpret_cast<const f32x4_t*>(&sD[buf][qb]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int e = 4 * e4 + r;
            float pv = exp2f(fmaf(s[c][e], p.scale_log2, -lq[r]));
            if (need_mask) {
              const int q = q0 + qb + r;
              if (mykv > q || q >= L || mykv >= L) pv = 0.f;
            }
            s[c][e] = pv;
            dp[c][e] = pv * (dp[c][e] - dq4[r]);
          }
        }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4_t pf = pack_half(s[ks >> 1], ks & 1);
        const u32x4_t df = pack_half(dp[ks >> 1], ks & 1);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const int off = (32 * dt + l32) * (QT + 8) + 16 * ks + 4 * h;
          dvt[dt] = mfma32(ld_pair8(sOt + off), pf, dvt[dt]);
          dkt[dt] = mfma32(ld_pair8(sQt + off), df, dkt[dt]);
        }
      }
    }
    if (more) store_tile((it + 1) & 1);
    __syncthreads();
  }

  if (mykv >= L) return;
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
template <int DH>
__global__ __launch_bounds__(256, 1) void attn_dq_kernel(const FwdP p) {
  constexpr int DHP = DH + 8;
  constexpr int NKK = DH / 16, NDT = DH / 32;
  constexpr int STAGE = 2 * KT * DHP + DH * KTP;   // K, V, K^T
  __shared__ __attribute__((aligned(16))) bf16_t smem[2][STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  const float dlt = p.delta[sidx];

  // Loader: K and V natural (16-byte chunks), K^T via 8x8 register blocks.
  constexpr int KCH = KT * DH / 8 / 256;
  u32x4_t kreg[KCH], vreg[KCH], treg[8];
  const bool tact = tid < (KT / 8) * (DH / 8);
  const int tkb = tid % (KT / 8), tdb = tid / (KT / 8);
  auto load_tile = [&](int t) {
    const int kv0 = t * KT;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + 256 * i;
      const int row = c / (DH / 8), cc = c % (DH / 8);
      const int kv = kv0 + row;
      const bool ok = kv < L;
      kreg[i] = ok ? ld16(p.k + (tok0 + kv) * p.ldk + (int64_t)kvh * DH + 8 * cc) : zero4();
      vreg[i] = ok ? ld16(p.v + (tok0 + kv) * p.ldv + (int64_t)kvh * DH + 8 * cc) : zero4();
    }
    if (tact) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int kv = kv0 + 8 * tkb + r;
        treg[r] = kv < L ? ld16(p.k + (tok0 + kv) * p.ldk + (int64_t)kvh * DH + 8 * tdb)
                         : zero4();
      }
    }
  };
  auto store_tile = [&](int buf) {
    bf16_t* sK = smem[buf];
    bf16_t* sV = sK + KT * DHP;
    bf16_t* sKt = sV + KT * DHP;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + 256 * i;
      const int row = c / (DH / 8), cc = c % (DH / 8);
      st16(sK + row * DHP + 8 * cc, kreg[i]);
      st16(sV + row * DHP + 8 * cc, vreg[i]);
    }
    if (tact) {
      u32x4_t t8[8];
      transpose8x8(treg, t8);
#pragma unroll
      for (int c = 0; c < 8; ++c) st16(sKt + (8 * tdb + c) * KTP + 8 * tkb, t8[c]);
    }
  };

  f32x16_t dqt[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) dqt[dt][e] = 0.f;

  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const bool more = t + 1 < ntiles;
    if (more) load_tile(t + 1);
    if (t < my_tiles) {
      const bf16_t* sK = smem[t & 1];
      const bf16_t* sV = sK + KT * DHP;
      const bf16_t* sKt = sV + KT * DHP;
      const int kv0 = t * KT;
      f32x16_t s[2], dp[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int e = 0; e < 16; ++e) { s[c][e] = 0.f; dp[c][e] = 0.f; }
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const int off = (32 * c + l32) * DHP + 16 * kk + 8 * h;
          s[c] = mfma32(ld16(sK + off), qf[kk], s[c]);
          dp[c] = mfma32(ld16(sV + off), of[kk], dp[c]);
        }
      }
      const bool need_mask = (kv0 + KT - 1 > qw0) || (kv0 + KT > L);
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float pv = exp2f(fmaf(s[c][e], p.scale_log2, -lse2));
          if (need_mask) {
            const int kv = kv0 + 32 * c + 8 * (e >> 2) + 4 * h + (e & 3);
            if (kv > qrow || kv >= L) pv = 0.f;
          }
          dp[c][e] = pv * (dp[c][e] - dlt);
        }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4_t df = pack_half(dp[ks >> 1], ks & 1);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          dqt[dt] = mfma32(ld_pair8(sKt + (32 * dt + l32) * KTP + 16 * ks + 4 * h), df,
                           dqt[dt]);
      }
    }
    if (more) store_tile((t + 1) & 1);
    __syncthreads();
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
  return p;
}

}  // namespace

hipError_t attn_fwd_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.B <= 0 || a.L <= 0) return hipSuccess;
  const FwdP p = make_params(a);
  const int QB = 32 * p.rb;
  dim3 grid((unsigned)(p.B * p.h_kv * (p.G / p.hb)), (unsigned)cdiv(p.L, QB));
  if (a.d_h == 128)
    hipLaunchKernelGGL(attn_fwd_kernel<128>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(attn_fwd_kernel<64>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t attn_bwd_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.B <= 0 || a.L <= 0) return hipSuccess;
  const FwdP p = make_params(a);
  const int64_t dthreads = (int64_t)p.B * p.L * p.h_q * (a.d_h / 8);
  dim3 dgrid((unsigned)cdiv(dthreads, 256));
  dim3 kgrid((unsigned)(p.B * p.h_kv), (unsigned)cdiv(p.L, 128));
  const int QB = 32 * p.rb;
  dim3 qgrid((unsigned)(p.B * p.h_kv * (p.G / p.hb)), (unsigned)cdiv(p.L, QB));
  if (a.d_h == 128) {
    hipLaunchKernelGGL(attn_delta_kernel<128>, dgrid, dim3(256), 0, s, p, a.delta);
    hipLaunchKernelGGL(attn_dkdv_kernel<128>, kgrid, dim3(256), 0, s, p);
    hipLaunchKernelGGL(attn_dq_kernel<128>, qgrid, dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL(attn_delta_kernel<64>, dgrid, dim3(256), 0, s, p, a.delta);
    hipLaunchKernelGGL(attn_dkdv_kernel<64>, kgrid, dim3(256), 0, s, p);
    hipLaunchKernelGGL(attn_dq_kernel<64>, qgrid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace q3l
