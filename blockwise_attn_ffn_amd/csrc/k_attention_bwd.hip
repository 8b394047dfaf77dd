// Attention backward (gfx950): dQ, dK and dV of A = softmax(Q K^T / sqrt(d_k)) V
// per (sequence, head), given dA = dO, the forward's output O and its saved
// per-row statistic lse.
//
// "Blockwise Parallel Transformer — BPT" (aicassindra.com), section "The backward
// pass": the forward keeps only each row's softmax statistics, and every block
// recomputes its scores and softmax from them and accumulates gradients at once;
// the FlashAttention paragraph of the transformer-cost page (raminaeye.github.io):
// the backward keeps the per-row statistics and recomputes the tiles. Per block:
//   P  = exp(S - lse)            S = Q K^T / sqrt(d_k), masked as in the forward
//   dV += P^T dO                 dP = dO V^T
//   dS = P * (dP - D)            D = rowsum(dO * O) per query row
//   dQ += dS K / sqrt(d_k)       dK += dS^T Q / sqrt(d_k)
//
// Two kernels, no atomics: one per query block for dQ (one lane per query row, as
// in the forward: S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T) and one per
// key/value block for dK and dV (one lane per key: S = Q K^T, dP = dO V^T,
// dV^T += dO^T P, dK^T += Q^T dS). The operands are first copied from the row-major
// inputs into the matrix-core fragment layouts the products read (bpt_device.hpp):
//   rows-B: B fragments over [token rows, d] (the forward's Q layout);
//   rows-A: per (sequence, head) A fragments over [tokens (pi order), d_k] (K's);
//   cols-A: per (sequence, head) A fragments over [d_k (pi order), tokens] (V^T's).
#include "bpt_device.hpp"
#include "bpt_launch.hpp"

namespace bpt {

enum BwdPackMode { kRowsB = 0, kRowsA = 1, kColsA = 2 };

// One thread per 8 elements of the destination. Padded token positions (pos >= N)
// are written as zeros.
__global__ __launch_bounds__(256) void bwd_pack_kernel(const bf16* __restrict__ src,
                                                       bf16* __restrict__ dst, int mode, int B,
                                                       int N, int Np, int H, int dk, int d) {
  const long long s = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long total = (long long)B * Np * (d / 8);
  if (s >= total) return;
  float v[8];
  if (mode != kColsA) {
    // 8 consecutive features of one token
    const int cpr = d / 8;
    const long long prow = s / cpr;
    const int col = (int)(s - prow * cpr) * 8;
    const int b = (int)(prow / Np), pos = (int)(prow - (long long)b * Np);
    if (pos < N) load8_f32(src + ((size_t)b * N + pos) * d + col, v);
    else
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
    size_t frag;
    int slot;
    if (mode == kRowsB) {
      frag = (size_t)(prow >> 5) * (d / 16) + (col >> 4);
      slot = 32 * ((col >> 3) & 1) + (int)(prow & 31);
    } else {
      const int h = col / dk, j = col - h * dk;
      frag = (((size_t)b * H + h) * (Np / 32) + (pos >> 5)) * (dk / 16) + (j >> 4);
      slot = 32 * ((j >> 3) & 1) + pi_row(pos & 31);
    }
    st_packed(dst + frag * kFragElems, slot, v);
  } else {
    // one feature of 8 consecutive tokens (a gather down the column)
    const int ppr = Np / 8;                       // 8-token groups per sequence
    const long long t = s / ppr;                  // (b, column)
    const int g8 = (int)(s - t * ppr);
    const int b = (int)(t / d), col = (int)(t - (long long)b * d);
    const int h = col / dk, j = col - h * dk;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int pos = g8 * 8 + e;
      v[e] = pos < N ? (float)src[((size_t)b * N + pos) * d + col] : 0.f;
    }
    const size_t frag = (((size_t)b * H + h) * (dk / 32) + (j >> 5)) * (Np / 16) + (g8 >> 1);
    const int slot = 32 * (g8 & 1) + pi_row(j & 31);
    st_packed(dst + frag * kFragElems, slot, v);
  }
}

// D[(b H + h) N + pos] = sum over the head's features of dO * O (fp32).
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(const bf16* __restrict__ dO,
                                                         const bf16* __restrict__ O,
                                                         float* __restrict__ D, int B, int N, int H,
                                                         int dk, int d) {
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;   // (b, h, pos)
  if (t >= (long long)B * H * N) return;
  const int pos = (int)(t % N);
  const long long bh = t / N;
  const int h = (int)(bh % H), b = (int)(bh / H);
  const size_t base = ((size_t)b * N + pos) * d + (size_t)h * dk;
  float acc = 0.f;
  for (int j = 0; j < dk; j += 8) {
    float x[8], y[8];
    load8_f32(dO + base + j, x);
    load8_f32(O + base + j, y);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(x[e], y[e], acc);
  }
  D[t] = acc;
}

struct BwdArgs {
  const bf16 *qB, *doB, *kA, *vA, *kT;            // dQ kernel operands
  const bf16 *kB, *vB, *qA, *doA, *qT, *doT;      // dK / dV kernel operands
  const float* lse;                               // [B, H, N], natural log
  const float* D;                                 // [B, H, N]
  float *dq, *dk, *dv;                            // [B N, d] row-major
  int B, N, Np, H, d, causal;
  float scale_log2e, scale;                       // log2(e) / sqrt(d_k), 1 / sqrt(d_k)
};

// dQ: one workgroup of 4 waves per (sequence, head, 128-row query block); one lane
// per query row. Key/value blocks of 64 keys are copied into LDS (K and V as A
// fragments over keys, K^T as A fragments over features), two stages.
template <int DK>
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(BwdArgs g) {
  using O = Op<bf16>;
  using F = O::frag;
  constexpr int BQ = 128, BKV = 64, FB = 1024;
  constexpr int KSD = DK / 16, KT = BKV / 32, DT = DK / 32, KK = BKV / 16;
  constexpr int KFR = KT * KSD;                 // K (and V) fragments per block
  constexpr int TFR = DT * KK;                  // K^T fragments per block
  constexpr int NFR = 2 * KFR + TFR;
  constexpr int CPW = NFR / 4;
  static_assert(NFR % 4 == 0, "copies per wave");
  __shared__ __align__(16) unsigned char lds0[NFR * FB];
  __shared__ __align__(16) unsigned char lds1[NFR * FB];

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rho = lane & 31, hf = lane >> 5;
  const int N = g.N, Np = g.Np, H = g.H, d = g.d;
  const int nqb = (N + BQ - 1) / BQ;
  const int bh = blockIdx.x / nqb, qb = blockIdx.x - bh * nqb;
  const int b = bh / H, h = bh - b * H;
  const int kend = g.causal ? (min(qb * BQ + BQ, N) - 1) / BKV + 1 : (N + BKV - 1) / BKV;
  const int wave_q_first = qb * BQ + wave * 32, qpos = wave_q_first + rho;

  auto issue = [&](int kb, unsigned char* buf) __attribute__((always_inline)) {
    const int kv0 = kb * BKV;
#pragma unroll
    for (int q = 0; q < CPW; ++q) {
      const int f = wave * CPW + q;
      const bf16* src;
      if (f < KFR) {
        src = g.kA + (((size_t)bh * (Np / 32) + kv0 / 32) * KSD + f) * kFragElems;
      } else if (f < 2 * KFR) {
        src = g.vA + (((size_t)bh * (Np / 32) + kv0 / 32) * KSD + (f - KFR)) * kFragElems;
      } else {
        const int ff = f - 2 * KFR, dt = ff / KK, kk = ff - dt * KK;
        src = g.kT + (((size_t)bh * DT + dt) * (Np / 16) + kv0 / 16 + kk) * kFragElems;
      }
      dma16(src + lane * 8, buf + f * FB);
    }
  };

  // this wave's Q and dO (B fragments over its 32 query rows) and row statistics
  F qf[KSD], of[KSD];
  {
    const size_t fr = (size_t)((b * Np + wave_q_first) >> 5) * (d / 16) + h * KSD;
#pragma unroll
    for (int kk = 0; kk < KSD; ++kk) {
      qf[kk] = ld_packed(g.qB + (fr + kk) * kFragElems, lane);
      of[kk] = ld_packed(g.doB + (fr + kk) * kFragElems, lane);
    }
  }
  const bool live = qpos < N;
  const float lse2 = live ? g.lse[(size_t)bh * N + qpos] * 1.4426950408889634f : 0.f;
  const float Dq = live ? g.D[(size_t)bh * N + qpos] : 0.f;
  f32x16 dq[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) dq[t] = f32x16{};

  auto visit = [&](int kb, const unsigned char* buf) __attribute__((always_inline)) {
    const int kv0 = kb * BKV;
    if (g.causal && kv0 > wave_q_first + 31) return;   // every key of the block is later
    f32x16 s[KT], dp[KT];
#pragma unroll
    for (int t = 0; t < KT; ++t) { s[t] = f32x16{}; dp[t] = f32x16{}; }
#pragma unroll
    for (int kk = 0; kk < KSD; ++kk)
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        O::mma(s[t], ld_packed(reinterpret_cast<const bf16*>(buf + (t * KSD + kk) * FB), lane), qf[kk]);
        O::mma(dp[t], ld_packed(reinterpret_cast<const bf16*>(buf + (KFR + t * KSD + kk) * FB), lane),
               of[kk]);
      }
    // register i of tile t holds key kv0 + t*32 + (i&8)*2 + 8hf + (i&7)
    const int lim = (g.causal ? min(qpos, N - 1) : N - 1) - kv0 - 8 * hf;
    F dsf[KK];
#pragma unroll
    for (int t = 0; t < KT; ++t) {
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = 8 * gg + e;
          const bool vis = live && (t * 32 + (i & 8) * 2 + (i & 7) <= lim);
          const float p = vis ? fast_exp2(fmaf(s[t][i], g.scale_log2e, -lse2)) : 0.f;
          v[e] = p * (dp[t][i] - Dq);
        }
        dsf[2 * t + gg] = O::from_f32(v);
      }
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int t = 0; t < DT; ++t)
        O::mma(dq[t], ld_packed(reinterpret_cast<const bf16*>(buf + (2 * KFR + t * KK + kk) * FB), lane),
               dsf[kk]);
  };

  issue(0, lds0);
  for (int kb = 0; kb < kend; kb += 2) {
    wait_vmem();
    __syncthreads();                     // stage 0 landed; stage 1 is free
    if (kb + 1 < kend) issue(kb + 1, lds1);
    visit(kb, lds0);
    if (kb + 1 >= kend) break;
    wait_vmem();
    __syncthreads();                     // stage 1 landed; stage 0 is free
    if (kb + 2 < kend) issue(kb + 2, lds0);
    visit(kb + 1, lds1);
  }
  // register group gg of feature tile t holds features t*32 + 16gg + 8hf + [0, 8)
  if (live) {
    float* out = g.dq + ((size_t)b * N + qpos) * d + (size_t)h * DK;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = dq[t][8 * gg + e] * g.scale;
        store8_f32(out + t * 32 + 16 * gg + 8 * hf, v);
      }
  }
}

// dK, dV: one workgroup of 4 waves per (sequence, head, 128-key block); one lane per
// key. Query blocks of 64 rows are copied into LDS (Q and dO as A fragments over
// queries, Q^T and dO^T as A fragments over features), two stages.
template <int DK>
__global__ __launch_bounds__(256, 1) void bwd_dkv_kernel(BwdArgs g) {
  using O = Op<bf16>;
  using F = O::frag;
  constexpr int BK = 128, BQS = 64, FB = 1024;
  constexpr int KSD = DK / 16, QT = BQS / 32, DT = DK / 32, QK = BQS / 16;
  constexpr int AFR = QT * KSD;                 // Q (and dO) fragments per block
  constexpr int TFR = DT * QK;                  // Q^T (and dO^T) fragments per block
  constexpr int NFR = 2 * AFR + 2 * TFR;
  constexpr int CPW = NFR / 4;
  static_assert(NFR % 4 == 0, "copies per wave");
  __shared__ __align__(16) unsigned char lds0[NFR * FB];
  __shared__ __align__(16) unsigned char lds1[NFR * FB];

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rho = lane & 31, hf = lane >> 5;
  const int N = g.N, Np = g.Np, H = g.H, d = g.d;
  const int nkb = (N + BK - 1) / BK;
  const int bh = blockIdx.x / nkb, kbk = blockIdx.x - bh * nkb;
  const int b = bh / H, h = bh - b * H;
  const int wave_k_first = kbk * BK + wave * 32, kpos = wave_k_first + rho;
  const int nqs = (N + BQS - 1) / BQS;
  const int qs_begin = g.causal ? (kbk * BK) / BQS : 0;

  auto issue = [&](int qs, unsigned char* buf) __attribute__((always_inline)) {
    const int q0 = qs * BQS;
#pragma unroll
    for (int q = 0; q < CPW; ++q) {
      const int f = wave * CPW + q;
      const bf16* src;
      if (f < 2 * AFR) {
        const bf16* base = f < AFR ? g.qA : g.doA;
        const int ff = f < AFR ? f : f - AFR;
        src = base + (((size_t)bh * (Np / 32) + q0 / 32) * KSD + ff) * kFragElems;
      } else {
        const int f2 = f - 2 * AFR;
        const bf16* base = f2 < TFR ? g.qT : g.doT;
        const int ff = f2 < TFR ? f2 : f2 - TFR, dt = ff / QK, kk = ff - dt * QK;
        src = base + (((size_t)bh * DT + dt) * (Np / 16) + q0 / 16 + kk) * kFragElems;
      }
      dma16(src + lane * 8, buf + f * FB);
    }
  };

  // this wave's K and V (B fragments over its 32 keys)
  F kf[KSD], vf[KSD];
  {
    const size_t fr = (size_t)((b * Np + wave_k_first) >> 5) * (d / 16) + h * KSD;
#pragma unroll
    for (int kk = 0; kk < KSD; ++kk) {
      kf[kk] = ld_packed(g.kB + (fr + kk) * kFragElems, lane);
      vf[kk] = ld_packed(g.vB + (fr + kk) * kFragElems, lane);
    }
  }
  f32x16 dkacc[DT], dvacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) { dkacc[t] = f32x16{}; dvacc[t] = f32x16{}; }
  const float* lse_bh = g.lse + (size_t)bh * N;
  const float* D_bh = g.D + (size_t)bh * N;

  auto visit = [&](int qs, const unsigned char* buf) __attribute__((always_inline)) {
    const int q0 = qs * BQS;
    if (g.causal && wave_k_first > q0 + BQS - 1) return;   // every query of the block is earlier
    f32x16 s[QT], dp[QT];
#pragma unroll
    for (int t = 0; t < QT; ++t) { s[t] = f32x16{}; dp[t] = f32x16{}; }
#pragma unroll
    for (int kk = 0; kk < KSD; ++kk)
#pragma unroll
      for (int t = 0; t < QT; ++t) {
        O::mma(s[t], ld_packed(reinterpret_cast<const bf16*>(buf + (t * KSD + kk) * FB), lane), kf[kk]);
        O::mma(dp[t], ld_packed(reinterpret_cast<const bf16*>(buf + (AFR + t * KSD + kk) * FB), lane),
               vf[kk]);
      }
    // register i of tile t holds query q0 + t*32 + (i&8)*2 + 8hf + (i&7); lane holds key kpos
    F pf[QK], dsf[QK];
#pragma unroll
    for (int t = 0; t < QT; ++t) {
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        const int qfirst = q0 + t * 32 + 16 * gg + 8 * hf;   // 8 consecutive queries
        float l8[8], d8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int qq = qfirst + e;
          l8[e] = qq < N ? lse_bh[qq] * 1.4426950408889634f : 0.f;
          d8[e] = qq < N ? D_bh[qq] : 0.f;
        }
        float pv[8], dv8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int qq = qfirst + e;
          const bool vis = kpos < N && qq < N && !(g.causal && kpos > qq);
          const float p = vis ? fast_exp2(fmaf(s[t][8 * gg + e], g.scale_log2e, -l8[e])) : 0.f;
          pv[e] = p;
          dv8[e] = p * (dp[t][8 * gg + e] - d8[e]);
        }
        pf[2 * t + gg] = O::from_f32(pv);
        dsf[2 * t + gg] = O::from_f32(dv8);
      }
    }
#pragma unroll
    for (int kk = 0; kk < QK; ++kk)
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        O::mma(dvacc[t],
               ld_packed(reinterpret_cast<const bf16*>(buf + (2 * AFR + TFR + t * QK + kk) * FB), lane),
               pf[kk]);
        O::mma(dkacc[t], ld_packed(reinterpret_cast<const bf16*>(buf + (2 * AFR + t * QK + kk) * FB), lane),
               dsf[kk]);
      }
  };

  if (qs_begin < nqs) {
    issue(qs_begin, lds0);
    for (int qs = qs_begin; qs < nqs; qs += 2) {
      wait_vmem();
      __syncthreads();
      if (qs + 1 < nqs) issue(qs + 1, lds1);
      visit(qs, lds0);
      if (qs + 1 >= nqs) break;
      wait_vmem();
      __syncthreads();
      if (qs + 2 < nqs) issue(qs + 2, lds0);
      visit(qs + 1, lds1);
    }
  }
  // register group gg of feature tile t holds features t*32 + 16gg + 8hf + [0, 8)
  if (kpos < N) {
    float* ok = g.dk + ((size_t)b * N + kpos) * d + (size_t)h * DK;
    float* ov = g.dv + ((size_t)b * N + kpos) * d + (size_t)h * DK;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        float v[8], w[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          v[e] = dkacc[t][8 * gg + e] * g.scale;
          w[e] = dvacc[t][8 * gg + e];
        }
        store8_f32(ok + t * 32 + 16 * gg + 8 * hf, v);
        store8_f32(ov + t * 32 + 16 * gg + 8 * hf, w);
      }
  }
}

namespace {

int pack(const bf16* src, bf16* dst, int mode, const AttnBwdLaunch& L, hipStream_t s, char* err,
         size_t n) {
  const long long total = (long long)L.batch * L.seq_pad * (L.d_model / 8);
  hipLaunchKernelGGL(bwd_pack_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, src, dst,
                     mode, L.batch, L.seq_len, L.seq_pad, L.n_heads, L.d_head, L.d_model);
  return check_launch("bwd_pack", err, n);
}

template <int DK>
int run_bwd(const AttnBwdLaunch& L, hipStream_t s, char* err, size_t n) {
  BwdArgs g{};
  const bf16* q = static_cast<const bf16*>(L.q);
  const bf16* k = static_cast<const bf16*>(L.k);
  const bf16* v = static_cast<const bf16*>(L.v);
  const bf16* dO = static_cast<const bf16*>(L.dout);
  bf16* P[kAttnBwdPacked];                          // packed copies in the workspace
  for (int i = 0; i < kAttnBwdPacked; ++i) P[i] = static_cast<bf16*>(L.packed[i]);
  if (pack(q, P[0], kRowsB, L, s, err, n) || pack(dO, P[1], kRowsB, L, s, err, n) ||
      pack(k, P[2], kRowsA, L, s, err, n) || pack(v, P[3], kRowsA, L, s, err, n) ||
      pack(k, P[4], kColsA, L, s, err, n) || pack(k, P[5], kRowsB, L, s, err, n) ||
      pack(v, P[6], kRowsB, L, s, err, n) || pack(q, P[7], kRowsA, L, s, err, n) ||
      pack(dO, P[8], kRowsA, L, s, err, n) || pack(q, P[9], kColsA, L, s, err, n) ||
      pack(dO, P[10], kColsA, L, s, err, n))
    return 1;
  const long long rows = (long long)L.batch * L.n_heads * L.seq_len;
  hipLaunchKernelGGL(bwd_rowdot_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, dO,
                     static_cast<const bf16*>(L.out), L.D, L.batch, L.seq_len, L.n_heads, L.d_head,
                     L.d_model);
  if (check_launch("bwd_rowdot", err, n)) return 1;
  g.qB = P[0]; g.doB = P[1]; g.kA = P[2]; g.vA = P[3]; g.kT = P[4];
  g.kB = P[5]; g.vB = P[6]; g.qA = P[7]; g.doA = P[8]; g.qT = P[9]; g.doT = P[10];
  g.lse = L.lse;
  g.D = L.D;
  g.dq = L.dq; g.dk = L.dk; g.dv = L.dv;
  g.B = L.batch; g.N = L.seq_len; g.Np = L.seq_pad; g.H = L.n_heads; g.d = L.d_model;
  g.causal = L.causal;
  g.scale = 1.0f / sqrtf((float)DK);
  g.scale_log2e = 1.4426950408889634f * g.scale;
  const int nqb = (L.seq_len + 127) / 128, nkb = (L.seq_len + 127) / 128;
  const int bhs = L.batch * L.n_heads;
  hipLaunchKernelGGL(bwd_dq_kernel<DK>, dim3(bhs * nqb), dim3(256), 0, s, g);
  if (check_launch("bwd_dq", err, n)) return 1;
  hipLaunchKernelGGL(bwd_dkv_kernel<DK>, dim3(bhs * nkb), dim3(256), 0, s, g);
  return check_launch("bwd_dkv", err, n);
}

}  // namespace

int launch_attention_bwd(const AttnBwdLaunch& L, void* stream, char* err, size_t n) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (L.d_head == 64) return run_bwd<64>(L, s, err, n);
  if (L.d_head == 128) return run_bwd<128>(L, s, err, n);
  set_err(err, n, "attention backward: head size %s%d unsupported (64 or 128)", "", L.d_head);
  return 1;
}

}  // namespace bpt
