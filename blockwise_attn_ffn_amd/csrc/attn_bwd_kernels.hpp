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
// dV^T += dO^T P, dK^T += Q^T dS). Operands whose matrix-core fragments hold 8
// consecutive features of one token (bpt_device.hpp) are read straight from the
// row-major inputs. The products that contract over tokens (K^T dS^T, dO^T P,
// Q^T dS) need 8 consecutive tokens of one feature per lane: for those, K, Q and
// dO are first transposed into packed fragments in the workspace ("cols-A": per
// (sequence, head) A fragments over [d_k (pi order), tokens], zero past seq_len).
// A first kernel also writes, per (sequence, head) and padded to Np rows,
// -D = -rowsum(dO * O) (negated, so that it can start the dP accumulator) and
// lse * log2(e) (+inf past seq_len, so that padded query rows get P = 0).
//
// The kernels are templates instantiated by the translation units that launch
// them: k_attention_bwd.hip (compiled with the products kept in VGPRs) and
// k_attention_bwd_dkv.hip (the d_k 128 dK / dV kernel, compiled without).
#pragma once

#include "attn_pack.hpp"
#include "bpt_device.hpp"
#include "bpt_launch.hpp"

namespace bpt {

constexpr float kLog2e = 1.4426950408889634f;

// Row statistics. One group of DK/8 consecutive threads per (token row, head),
// each thread 8 consecutive features, so a wave reads whole rows contiguously:
//   Dp[bh * Np + pos] = -(sum over the head's features of dO * O)   (0 past N)
//   L2[bh * Np + pos] = lse * log2(e)                          (+inf past N)
template <int DK>
__global__ __launch_bounds__(256) void bwd_stats_kernel(const bf16* __restrict__ dO,
                                                        const bf16* __restrict__ O,
                                                        const float* __restrict__ lse,
                                                        float* __restrict__ Dp,
                                                        float* __restrict__ L2, int B, int N,
                                                        int Np, int H) {
  constexpr int CH = DK / 8;
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  // B * Np * H * CH is a multiple of 256 (Np is a multiple of 128): no partial group
  const int c = (int)(t % CH);
  const long long rh = t / CH;
  const int h = (int)(rh % H);
  const long long row = rh / H;
  const int b = (int)(row / Np), pos = (int)(row - (long long)b * Np);
  float acc = 0.f;
  if (pos < N) {
    const size_t off = ((size_t)b * N + pos) * (size_t)(H * DK) + (size_t)h * DK + c * 8;
    float x[8], y[8];
    load8_f32(dO + off, x);
    load8_f32(O + off, y);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(x[e], y[e], acc);
  }
#pragma unroll
  for (int o = CH / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (c == 0) {
    const size_t i = ((size_t)b * H + h) * Np + pos;
    Dp[i] = -acc;
    L2[i] = pos < N ? lse[((size_t)b * H + h) * N + pos] * kLog2e : __builtin_inff();
  }
}

template <bool B> struct BoolTag { static constexpr bool value = B; };
struct RuntimeTag {};   // decide the masking inside the body, around the softmax only

struct BwdArgs {
  const bf16 *q, *k, *v, *dout;                   // row-major [B N, d]
  const bf16 *kT, *qT, *doT;                      // cols-A fragments per (sequence, head)
  const float *L2, *Dp;                           // [B H, Np]: lse log2 e, -D
  float *dq, *dk, *dv;                            // [B N, d] row-major
  int B, N, Np, H, d, causal;
  int G, dkv, window, chunk;                      // key/value heads, their width, masks
  float scale_log2e, scale;                       // log2(e) / sqrt(d_k), 1 / sqrt(d_k)
};

// Visible keys [lo, hi] of query position p (the forward's masks; p past the end
// behaves as the last row). GENERAL instances only; the others are plain causal /
// unmasked with one key/value head per query head.
template <bool GENERAL>
__device__ inline int bwd_key_hi(const BwdArgs& g, int p) {
  const int pc = min(p, g.N - 1);
  if (!g.causal) return g.N - 1;
  if constexpr (GENERAL) return g.chunk ? min((pc / g.chunk + 1) * g.chunk, g.N) - 1 : pc;
  return pc;
}
template <bool GENERAL>
__device__ inline int bwd_key_lo(const BwdArgs& g, int p) {
  if constexpr (GENERAL) return g.window ? max(0, min(p, g.N - 1) - g.window + 1) : 0;
  return 0;
}

// Lane's fragment of a B operand over token rows from row-major X: row `pos`
// (zero past N), features f0 + [0, 8).
__device__ inline bf16x8 ld_row_frag(const bf16* X, int b, int pos, int N, int d, int f0) {
  if (pos >= N) return bf16x8{};
  return *reinterpret_cast<const bf16x8*>(X + ((size_t)b * N + pos) * d + f0);
}

// dQ: one workgroup of NW waves per (sequence, head, 32 NW-row query block); one
// lane per query row. Key/value blocks of 64 keys are copied into LDS (K and V as A
// fragments over keys, straight from the row-major inputs; K^T as A fragments over
// features from the transposed copy), two stages shared by all NW waves.
template <int DK, int NW, bool GENERAL>
__global__ __launch_bounds__(64 * NW, 1) void bwd_dq_kernel(BwdArgs g) {
  using O = Op<bf16>;
  using F = O::frag;
  constexpr int BQ = 32 * NW, BKV = 64, FB = 1024;
  constexpr int KSD = DK / 16, KT = BKV / 32, DT = DK / 32, KK = BKV / 16;
  constexpr int KFR = KT * KSD;                 // K (and V) fragments per block
  constexpr int TFR = DT * KK;                  // K^T fragments per block
  constexpr int NFR = 2 * KFR + TFR;
  constexpr int CPW = NFR / NW;
  static_assert(KFR % NW == 0 && TFR % NW == 0, "copies per wave");
  __shared__ __align__(16) unsigned char lds0[NFR * FB];
  __shared__ __align__(16) unsigned char lds1[NFR * FB];

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rho = lane & 31, hf = lane >> 5;
  const int N = g.N, Np = g.Np, H = g.H, d = g.d;
  const int nqb = (N + BQ - 1) / BQ;
  const int bh = blockIdx.x / nqb, qb = nqb - 1 - (int)(blockIdx.x - bh * nqb);   // longest first
  const int b = bh / H, h = bh - b * H;
  const int gk = GENERAL ? h / (H / g.G) : h;   // key/value head read by this query head
  const int bg = GENERAL ? b * g.G + gk : bh;
  const int dkv = GENERAL ? g.dkv : d;
  const int kbeg = bwd_key_lo<GENERAL>(g, qb * BQ) / BKV;
  const int kend = bwd_key_hi<GENERAL>(g, qb * BQ + BQ - 1) / BKV + 1;
  const int wave_q_first = qb * BQ + wave * 32, qpos = wave_q_first + rho;
  const int fcol = h * DK + 8 * hf;             // this lane's feature offset in a row
  const int fkv = gk * DK + 8 * hf;             // the same in a K / V row
  const int prho = pi_row(rho);
  static_assert(KSD % NW == 0 && NW % KK == 0, "copy slots");

  // Copy slot q of wave w moves fragment NW q + w of the stage, so that the kind of
  // copy (K, V or K^T) and its tile are the same in every wave: fixed at compile
  // time; the wave's own part of each address is a wave-uniform offset.
  auto issue = [&](int kb, unsigned char* buf) __attribute__((always_inline)) {
    const int kv0 = kb * BKV;
    size_t rowoff[KT];                            // this lane's key row in each 32-key tile
#pragma unroll
    for (int t = 0; t < KT; ++t) rowoff[t] = ((size_t)b * N + min(kv0 + t * 32 + prho, N - 1)) * dkv + fkv;
    // K^T fragment (dt, k-step) = (slot / KK, slot % KK); the wave adds (w / KK, w % KK)
    const bf16* kt_base =
        g.kT + (((size_t)bg * DT + wave / KK) * (Np / 16) + kv0 / 16 + wave % KK) * kFragElems + lane * 8;
#pragma unroll
    for (int q = 0; q < CPW; ++q) {
      const int f0 = NW * q;
      const bf16* src;
      if (f0 < 2 * KFR) {
        const int ff0 = f0 < KFR ? f0 : f0 - KFR, t = ff0 / KSD, kk = ff0 % KSD + wave;
        src = (f0 < KFR ? g.k : g.v) + rowoff[t] + kk * 16;
      } else {
        const int dt0 = (f0 - 2 * KFR) / KK;
        src = kt_base + (size_t)dt0 * (Np / 16) * kFragElems;
      }
      dma16(src, buf + (f0 + wave) * FB);
    }
  };

  // this wave's Q and dO (B fragments over its 32 query rows) and row statistics
  F qf[KSD], of[KSD];
#pragma unroll
  for (int kk = 0; kk < KSD; ++kk) {
    qf[kk] = ld_row_frag(g.q, b, qpos, N, d, fcol + kk * 16);
    of[kk] = ld_row_frag(g.dout, b, qpos, N, d, fcol + kk * 16);
  }
  // rows past N (the last block may reach beyond the padded Np rows): P = 0
  const bool live = qpos < N;
  const float l2 = live ? g.L2[(size_t)bh * Np + qpos] : __builtin_inff();
  const float nDq = live ? g.Dp[(size_t)bh * Np + qpos] : 0.f;   // -D
  f32x16 dq[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) dq[t] = f32x16{};

  auto visit = [&](int kb, const unsigned char* buf) __attribute__((always_inline)) {
    const int kv0 = kb * BKV;
    // no row of the wave sees a key of the block
    if (kv0 > bwd_key_hi<GENERAL>(g, wave_q_first + 31)) return;
    if (GENERAL && kv0 + BKV - 1 < bwd_key_lo<GENERAL>(g, wave_q_first)) return;
    const bool need_mask = kv0 + BKV - 1 > bwd_key_hi<GENERAL>(g, wave_q_first) ||
                           (GENERAL && kv0 < bwd_key_lo<GENERAL>(g, wave_q_first + 31));
    f32x16 s[KT], dp[KT];
    F dsf[KK];
    // register i of tile t holds key kv0 + t*32 + (i&8)*2 + 8hf + (i&7)
    const int lim = bwd_key_hi<GENERAL>(g, qpos) - kv0 - 8 * hf;
    const int lim_lo = bwd_key_lo<GENERAL>(g, qpos) - kv0 - 8 * hf;
    auto softmax_grad = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
      for (int t = 0; t < KT; ++t) {
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int i = 8 * gg + e;
            float p = fast_exp2(fmaf(s[t][i], g.scale_log2e, -l2));
            const int off = t * 32 + (i & 8) * 2 + (i & 7);
            if (decltype(masked)::value && (off > lim || (GENERAL && off < lim_lo))) p = 0.f;
            v[e] = p * (dp[t][i] + nDq);
          }
          dsf[2 * t + gg] = O::from_f32(v);
        }
      }
    };
    // The body branches around the softmax only: a body specialised per masking
    // mode (straight-line) holds more registers live and measured no faster.
    auto ld_a = [&](int f) __attribute__((always_inline)) {
      return ld_packed(reinterpret_cast<const bf16*>(buf + f * FB), lane);
    };
    auto body = [&](RuntimeTag) __attribute__((always_inline)) {
#pragma unroll
      for (int t = 0; t < KT; ++t) { s[t] = f32x16{}; dp[t] = f32x16{}; }
      // products in the order written, each LDS read four products ahead
      constexpr int DD = 4, N1 = 2 * KT * KSD, N2 = DT * KK;
      // first: (kk, t, S or dP) -> fragment (S: t KSD + kk, dP: KFR + t KSD + kk)
      auto f1 = [](int x) { const int kk = x / (2 * KT), t = (x / 2) % KT; return (x & 1) * KFR + t * KSD + kk; };
      F ring[DD];
#pragma unroll
      for (int x = 0; x < DD; ++x) ring[x] = ld_a(f1(x));
#pragma unroll
      for (int x = 0; x < N1; ++x) {
        __builtin_amdgcn_sched_barrier(0);
        const F a = ring[x % DD];
        if (x + DD < N1) ring[x % DD] = ld_a(f1(x + DD));
        const int kk = x / (2 * KT), t = (x / 2) % KT;
        if (x & 1) O::mma(dp[t], a, of[kk]);
        else O::mma(s[t], a, qf[kk]);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (need_mask) softmax_grad(BoolTag<true>{});
      else softmax_grad(BoolTag<false>{});
      // then dQ^T: (kk, t) -> fragment 2 KFR + t KK + kk
#pragma unroll
      for (int x = 0; x < DD; ++x) ring[x] = ld_a(2 * KFR + (x % DT) * KK + x / DT);
#pragma unroll
      for (int x = 0; x < N2; ++x) {
        __builtin_amdgcn_sched_barrier(0);
        const F a = ring[x % DD];
        if (x + DD < N2) ring[x % DD] = ld_a(2 * KFR + ((x + DD) % DT) * KK + (x + DD) / DT);
        O::mma(dq[x % DT], a, dsf[x / DT]);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    body(RuntimeTag{});
  };

  issue(kbeg, lds0);
  for (int kb = kbeg; kb < kend; kb += 2) {
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

// dK, dV: one workgroup of NW waves per (sequence, head, 32 NW-key block); one lane
// per key. Query blocks of BQS rows are copied into LDS (Q and dO as A fragments
// over queries from the row-major inputs, Q^T and dO^T from the transposed copies,
// and the rows' statistics), two stages shared by all NW waves.
template <int DK, int NW, int BQS, bool GENERAL>
__global__ __launch_bounds__(64 * NW, 1) void bwd_dkv_kernel(BwdArgs g) {
  using O = Op<bf16>;
  using F = O::frag;
  constexpr int BK = 32 * NW, FB = 1024;
  constexpr int KSD = DK / 16, QT = BQS / 32, DT = DK / 32, QK = BQS / 16;
  constexpr int AFR = QT * KSD;                 // Q (and dO) fragments per block
  constexpr int TFR = DT * QK;                  // Q^T (and dO^T) fragments per block
  constexpr int NFR = 2 * AFR + 2 * TFR;
  constexpr int CPW = NFR / NW;
  constexpr int STAGE = (NFR + 1) * FB;         // + statistics: L2 then Dp, BQS floats each
  static_assert(AFR % NW == 0 && TFR % NW == 0, "copies per wave");
  __shared__ __align__(16) unsigned char lds0[STAGE];
  __shared__ __align__(16) unsigned char lds1[STAGE];

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rho = lane & 31, hf = lane >> 5;
  const int N = g.N, Np = g.Np, H = g.H, d = g.d;
  const int nkb = (N + BK - 1) / BK;
  // workgroup: (sequence, key/value head, key block); with grouped heads it sums
  // over the query heads of its group (GS of them), one run of query stages each
  const int G = GENERAL ? g.G : H, GS = GENERAL ? H / g.G : 1, dkv = GENERAL ? g.dkv : d;
  const int bg = blockIdx.x / nkb, kbk = blockIdx.x - bg * nkb;   // longest first under the mask
  const int b = bg / G, gk = bg - b * G;
  const int wave_k_first = kbk * BK + wave * 32, kpos = wave_k_first + rho;
  const int nqs = (N + BQS - 1) / BQS;
  // query stages that can see a key of the block: from the first query whose
  // visible range reaches the block's first key to the last one reaching its last
  int qs_begin = 0, qs_end = nqs;
  if (g.causal) {
    const int k0 = kbk * BK, k1 = min(k0 + BK, N) - 1;
    int q_first = k0;                                        // causal: q >= k
    if (GENERAL && g.chunk) q_first = k0 / g.chunk * g.chunk;   // the key's whole chunk
    qs_begin = q_first / BQS;
    if (GENERAL && g.window) qs_end = min(nqs, (k1 + g.window - 1) / BQS + 1);
  }
  const int nst = qs_end - qs_begin, n_it = GS * nst;
  const int fkv = gk * DK + 8 * hf;
  const int prho = pi_row(rho);
  static_assert(KSD % NW == 0 && NW % QK == 0, "copy slots");

  // Copy slot q of wave w moves fragment NW q + w of the stage (the kind of copy is
  // the same in every wave); wave 0 also copies the BQS rows' statistics.
  auto issue = [&](int it, unsigned char* buf) __attribute__((always_inline)) {
    const int hq = GENERAL ? gk * GS + it / nst : gk;
    const int q0 = (qs_begin + (GENERAL ? it % nst : it)) * BQS;
    const int bh = b * H + hq, fcol = hq * DK + 8 * hf;
    size_t rowoff[QT];                            // this lane's query row in each 32-row tile
#pragma unroll
    for (int t = 0; t < QT; ++t) rowoff[t] = ((size_t)b * N + min(q0 + t * 32 + prho, N - 1)) * d + fcol;
    // Q^T / dO^T fragment (dt, k-step) = (slot / QK, slot % QK); the wave adds (w / QK, w % QK)
    const size_t toff =
        (((size_t)bh * DT + wave / QK) * (Np / 16) + q0 / 16 + wave % QK) * kFragElems + lane * 8;
#pragma unroll
    for (int q = 0; q < CPW; ++q) {
      const int f0 = NW * q;
      const bf16* src;
      if (f0 < 2 * AFR) {
        const int ff0 = f0 < AFR ? f0 : f0 - AFR, t = ff0 / KSD, kk = ff0 % KSD + wave;
        src = (f0 < AFR ? g.q : g.dout) + rowoff[t] + kk * 16;
      } else {
        const int f2 = f0 - 2 * AFR;
        const int dt0 = (f2 < TFR ? f2 : f2 - TFR) / QK;
        src = (f2 < TFR ? g.qT : g.doT) + toff + (size_t)dt0 * (Np / 16) * kFragElems;
      }
      dma16(src, buf + (f0 + wave) * FB);
    }
    if (wave == 0) {
      // lanes [0, BQS/4): L2[q0, q0 + BQS), the next BQS/4 lanes: Dp; the rest repeat them
      const int l = lane % (BQS / 2);
      const float* st = (l < BQS / 4 ? g.L2 : g.Dp) + (size_t)bh * Np + q0 + 4 * (l % (BQS / 4));
      dma16(st, buf + NFR * FB);
    }
  };

  // this wave's K and V (B fragments over its 32 keys)
  F kf[KSD], vf[KSD];
#pragma unroll
  for (int kk = 0; kk < KSD; ++kk) {
    kf[kk] = ld_row_frag(g.k, b, kpos, N, dkv, fkv + kk * 16);
    vf[kk] = ld_row_frag(g.v, b, kpos, N, dkv, fkv + kk * 16);
  }
  f32x16 dkacc[DT], dvacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) { dkacc[t] = f32x16{}; dvacc[t] = f32x16{}; }

  auto visit = [&](int it, const unsigned char* buf) __attribute__((always_inline)) {
    const int q0 = (qs_begin + (GENERAL ? it % nst : it)) * BQS;
    // no query of the stage sees a key of the wave
    if (wave_k_first > bwd_key_hi<GENERAL>(g, q0 + BQS - 1)) return;
    if (GENERAL && wave_k_first + 31 < bwd_key_lo<GENERAL>(g, q0)) return;
    const bool need_mask = wave_k_first + 31 > bwd_key_hi<GENERAL>(g, q0) ||
                           (GENERAL && wave_k_first < bwd_key_lo<GENERAL>(g, q0 + BQS - 1));
    f32x16 s[QT], dp[QT];
    F pf[QK], dsf[QK];
    // register i of tile t holds query q0 + t*32 + (i&8)*2 + 8hf + (i&7); lane holds key kpos
    const float* st = reinterpret_cast<const float*>(buf + NFR * FB);
    auto softmax_grad = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
      for (int t = 0; t < QT; ++t) {
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
          const int qoff = t * 32 + 16 * gg + 8 * hf;          // 8 consecutive queries
          const float4 la = *reinterpret_cast<const float4*>(st + qoff);
          const float4 lb = *reinterpret_cast<const float4*>(st + qoff + 4);
          const float l8[8] = {la.x, la.y, la.z, la.w, lb.x, lb.y, lb.z, lb.w};
          float pv[8], dv8[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float p = fast_exp2(fmaf(s[t][8 * gg + e], g.scale_log2e, -l8[e]));
            if constexpr (decltype(masked)::value) {
              const int qq = q0 + qoff + e;
              if (GENERAL ? (kpos > bwd_key_hi<true>(g, qq) || kpos < bwd_key_lo<true>(g, qq))
                          : (g.causal && kpos > qq))
                p = 0.f;
            }
            pv[e] = p;
            dv8[e] = p * dp[t][8 * gg + e];   // dp holds dP - D
          }
          pf[2 * t + gg] = O::from_f32(pv);
          dsf[2 * t + gg] = O::from_f32(dv8);
        }
      }
    };
    // branching around the softmax only (as in dQ)
    auto body = [&](RuntimeTag) __attribute__((always_inline)) {
      // the dP accumulators start from -D of their rows: dP - D comes out of the products
#pragma unroll
      for (int t = 0; t < QT; ++t) {
        s[t] = f32x16{};
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
          const float4 da = *reinterpret_cast<const float4*>(st + BQS + t * 32 + 16 * gg + 8 * hf);
          const float4 db = *reinterpret_cast<const float4*>(st + BQS + t * 32 + 16 * gg + 8 * hf + 4);
          dp[t][8 * gg + 0] = da.x; dp[t][8 * gg + 1] = da.y; dp[t][8 * gg + 2] = da.z; dp[t][8 * gg + 3] = da.w;
          dp[t][8 * gg + 4] = db.x; dp[t][8 * gg + 5] = db.y; dp[t][8 * gg + 6] = db.z; dp[t][8 * gg + 7] = db.w;
        }
      }
#pragma unroll
      for (int kk = 0; kk < KSD; ++kk)
#pragma unroll
        for (int t = 0; t < QT; ++t) {
          O::mma(s[t], ld_packed(reinterpret_cast<const bf16*>(buf + (t * KSD + kk) * FB), lane), kf[kk]);
          O::mma(dp[t], ld_packed(reinterpret_cast<const bf16*>(buf + (AFR + t * KSD + kk) * FB), lane),
                 vf[kk]);
        }
      if (need_mask) softmax_grad(BoolTag<true>{});
      else softmax_grad(BoolTag<false>{});
#pragma unroll
      for (int kk = 0; kk < QK; ++kk)
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          O::mma(dvacc[t],
                 ld_packed(reinterpret_cast<const bf16*>(buf + (2 * AFR + TFR + t * QK + kk) * FB), lane),
                 pf[kk]);
          O::mma(dkacc[t],
                 ld_packed(reinterpret_cast<const bf16*>(buf + (2 * AFR + t * QK + kk) * FB), lane), dsf[kk]);
        }
    };
    body(RuntimeTag{});
  };

  if (n_it > 0) issue(0, lds0);
  for (int it = 0; it < n_it; it += 2) {
    wait_vmem();
    __syncthreads();
    if (it + 1 < n_it) issue(it + 1, lds1);
    visit(it, lds0);
    if (it + 1 >= n_it) break;
    wait_vmem();
    __syncthreads();
    if (it + 2 < n_it) issue(it + 2, lds0);
    visit(it + 1, lds1);
  }
  // register group gg of feature tile t holds features t*32 + 16gg + 8hf + [0, 8)
  if (kpos < N) {
    float* ok = g.dk + ((size_t)b * N + kpos) * dkv + (size_t)gk * DK;
    float* ov = g.dv + ((size_t)b * N + kpos) * dkv + (size_t)gk * DK;
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


// dK, dV split by gradient: one workgroup of 8 waves per (sequence, key/value head,
// 128-key block), two waves per 32 keys on one SIMD. Wave w < 4 (the P wave) forms
// S = Q K^T and P and accumulates dV^T += dO^T P; its partner w + 4 (the dS wave)
// forms dP = dO V^T for the same keys, dS = P * (dP - D) with the P handed over
// through LDS (bf16, in the accumulator layout), and accumulates dK^T += Q^T dS.
// Each wave holds one accumulator set and one of K, V, so the two fit on one SIMD.
// Every query stage takes two half steps separated by barriers:
//   first half:  P wave  S, P (exp2), P -> LDS     dS wave  dK^T += Q^T dS (previous stage)
//   second half: P wave  dV^T += dO^T P            dS wave  dP, dS
// so in each half one wave's matrix products run beside the other wave's vector
// work. Stage operands (Q, dO^T, dO, Q^T as A fragments, and the rows' lse and -D)
// are double-buffered per kind and copied by the LDS-DMA path a step ahead; Q^T is
// kept one half step longer, so its copy is issued at the middle barrier. Only the
// step barrier waits for copies.
template <int DK, int BQS, bool GENERAL>
__global__ __launch_bounds__(512, 1) void bwd_dkv_split_kernel(BwdArgs g) {
  using O = Op<bf16>;
  using F = O::frag;
  constexpr int NW = 8, BK = 128, FB = 1024;
  constexpr int KSD = DK / 16, QT = BQS / 32, DT = DK / 32, QK = BQS / 16;
  constexpr int AFR = QT * KSD;                 // Q (or dO) fragments per stage
  constexpr int TFR = DT * QK;                  // Q^T (or dO^T) fragments per stage
  static_assert(AFR % NW == 0 && TFR % NW == 0 && KSD % NW == 0 && NW % QK == 0, "copy slots");
  static_assert(BQS == 64, "statistics copy: one 16-byte slot per 4 rows of each statistic");
  // per kind and stage parity; st: lse log2 e then -D of the stage's rows (1 KB slot)
  __shared__ __align__(16) unsigned char qa0[AFR * FB], qa1[AFR * FB];     // Q
  __shared__ __align__(16) unsigned char da0[AFR * FB], da1[AFR * FB];     // dO
  __shared__ __align__(16) unsigned char qt0[TFR * FB], qt1[TFR * FB];     // Q^T
  __shared__ __align__(16) unsigned char dt0[TFR * FB], dt1[TFR * FB];     // dO^T
  __shared__ __align__(16) unsigned char st0[FB], st1[FB];
  __shared__ __align__(16) unsigned char px[4 * QK * FB];                 // P of the 4 P waves

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rho = lane & 31, hf = lane >> 5;
  const bool pwave = wave < 4;
  const int kg = wave & 3;                      // the wave pair's 32 keys
  const int N = g.N, Np = g.Np, H = g.H, d = g.d;
  const int nkb = (N + BK - 1) / BK;
  const int G = GENERAL ? g.G : H, GS = GENERAL ? H / g.G : 1, dkv = GENERAL ? g.dkv : d;
  const int bg = blockIdx.x / nkb, kbk = blockIdx.x - bg * nkb;
  const int b = bg / G, gk = bg - b * G;
  const int wave_k_first = kbk * BK + kg * 32, kpos = wave_k_first + rho;
  const int nqs = (N + BQS - 1) / BQS;
  int qs_begin = 0, qs_end = nqs;
  if (g.causal) {
    const int k0 = kbk * BK, k1 = min(k0 + BK, N) - 1;
    int q_first = k0;
    if (GENERAL && g.chunk) q_first = k0 / g.chunk * g.chunk;
    qs_begin = q_first / BQS;
    if (GENERAL && g.window) qs_end = min(nqs, (k1 + g.window - 1) / BQS + 1);
  }
  const int nst = qs_end - qs_begin, n_it = GS * nst;
  const int fkv = gk * DK + 8 * hf;
  const int prho = pi_row(rho);

  auto stage_q0 = [&](int it) __attribute__((always_inline)) {
    return (qs_begin + (GENERAL ? it % nst : it)) * BQS;
  };
  auto stage_bh = [&](int it) __attribute__((always_inline)) {
    return b * H + (GENERAL ? gk * GS + it / nst : gk);
  };
  // A fragments over the stage's query rows (32-row tile t, feature k-step kk) from
  // row-major X; copy slot q of wave w moves fragment NW q + w
  // Copy addresses are a wave-uniform base plus a per-lane byte offset fixed for the
  // whole kernel (rows inside the sequence: every stage but a ragged last one).
  const unsigned lane_row_b = (unsigned)(prho * d + 8 * hf) * 2u;   // row-major operand
  const unsigned lane_frag_b = (unsigned)lane * 16u;                // packed fragment
  auto issue_rows = [&](int it, const bf16* X, unsigned char* buf) __attribute__((always_inline)) {
    const int q0 = stage_q0(it), bh = stage_bh(it);
    const int fcol = (bh - b * H) * DK;
    if (q0 + BQS <= N) {
      const char* base = reinterpret_cast<const char*>(X + ((size_t)b * N + q0) * d + fcol + wave * 16);
#pragma unroll
      for (int q = 0; q < AFR / NW; ++q) {
        const int f0 = NW * q, t = f0 / KSD;
        dma16(base + (size_t)t * 32 * d * 2 + lane_row_b, buf + (f0 + wave) * FB);
      }
    } else {
#pragma unroll
      for (int q = 0; q < AFR / NW; ++q) {
        const int f0 = NW * q, t = f0 / KSD, kk = f0 % KSD + wave;
        const size_t row = (size_t)b * N + min(q0 + t * 32 + prho, N - 1);
        dma16(X + row * d + fcol + 8 * hf + kk * 16, buf + (f0 + wave) * FB);
      }
    }
  };
  // A fragments over features (32-feature tile, query k-step) from a transposed copy
  auto issue_cols = [&](int it, const bf16* XT, unsigned char* buf) __attribute__((always_inline)) {
    const int q0 = stage_q0(it), bh = stage_bh(it);
    const char* base = reinterpret_cast<const char*>(
        XT + (((size_t)bh * DT + wave / QK) * (Np / 16) + q0 / 16 + wave % QK) * kFragElems);
#pragma unroll
    for (int q = 0; q < TFR / NW; ++q) {
      const int f0 = NW * q, dt = f0 / QK;
      dma16(base + (size_t)dt * (Np / 16) * kFragElems * 2 + lane_frag_b, buf + (f0 + wave) * FB);
    }
  };
  // everything of stage it except Q^T; wave 0 copies the statistics (lanes 0-15:
  // lse log2 e of the 64 rows, lanes 16-31: -D; the other lanes repeat them)
  const float* stat_lane = ((lane & 31) < 16 ? g.L2 : g.Dp) + 4 * (lane & 15);
  auto issue_step = [&](int it, unsigned char* qa, unsigned char* da, unsigned char* dt,
                        unsigned char* st) __attribute__((always_inline)) {
    issue_rows(it, g.q, qa);
    issue_cols(it, g.doT, dt);
    issue_rows(it, g.dout, da);
    if (wave == 0) dma16(stat_lane + (size_t)stage_bh(it) * Np + stage_q0(it), st);
  };

  auto run = [&](auto role) __attribute__((always_inline)) {
    constexpr bool PW = decltype(role)::value;   // P wave or dS wave
    // the wave's K (P waves) or V (dS waves) as B fragments over its 32 keys
    F kvf[KSD];
#pragma unroll
    for (int kk = 0; kk < KSD; ++kk) kvf[kk] = ld_row_frag(PW ? g.k : g.v, b, kpos, N, dkv, fkv + kk * 16);
    f32x16 acc[DT];                               // dV^T (P waves) or dK^T (dS waves)
#pragma unroll
    for (int t = 0; t < DT; ++t) acc[t] = f32x16{};
    F pf[QK];                                     // P wave: P of the current stage
    F dsf[QK];                                    // dS wave: dS of the previous stage
    bool carry = false;                           // the held P / dS belongs to a live stage

    auto stage_live = [&](int q0) __attribute__((always_inline)) {
      if (wave_k_first > bwd_key_hi<GENERAL>(g, q0 + BQS - 1)) return false;
      if (GENERAL && wave_k_first + 31 < bwd_key_lo<GENERAL>(g, q0)) return false;
      return true;
    };
    // 8 consecutive rows' statistic (0: lse log2 e, 1: -D) from a stage's slot
    auto stat8 = [&](const unsigned char* st, int which, int qoff, float* v) __attribute__((always_inline)) {
      const float* p = reinterpret_cast<const float*>(st) + 64 * which + qoff;
      const float4 a = *reinterpret_cast<const float4*>(p);
      const float4 c = *reinterpret_cast<const float4*>(p + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = c.x; v[5] = c.y; v[6] = c.z; v[7] = c.w;
    };

    // c[t] += A(t, kk) B[kk] over all (kk, t), kk outer; A(t, kk) is the packed
    // fragment at base + (t * TS + kk * KS) KB; its LDS reads run four products ahead
    auto stream = [&](auto nt, auto nk, auto ts, auto ks, f32x16* c, const unsigned char* base,
                      const F* bfr) __attribute__((always_inline)) {
      constexpr int NT = decltype(nt)::value, NK = decltype(nk)::value;
      constexpr int TS = decltype(ts)::value, KS = decltype(ks)::value;
      constexpr int NN = NT * NK, DD = 4;
      auto ld = [&](int j) __attribute__((always_inline)) {
        return ld_packed(reinterpret_cast<const bf16*>(base + ((j % NT) * TS + (j / NT) * KS) * FB), lane);
      };
      F ring[DD];
#pragma unroll
      for (int j = 0; j < DD; ++j) ring[j] = ld(j);
#pragma unroll
      for (int j = 0; j < NN; ++j) {
        // the order as written: the scheduler would otherwise pull each read down
        // next to its product
        __builtin_amdgcn_sched_barrier(0);
        const F a = ring[j % DD];
        if (j + DD < NN) ring[j % DD] = ld(j + DD);
        O::mma(c[j % NT], a, bfr[j / NT]);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    using IQT = std::integral_constant<int, QT>;
    using IDT = std::integral_constant<int, DT>;
    using IKSD = std::integral_constant<int, KSD>;
    using IQK = std::integral_constant<int, QK>;
    using I1 = std::integral_constant<int, 1>;

    // first half, P wave: S = Q K^T, P = exp2(S log2e / sqrt(d_k) - lse log2e) -> pf, px.
    // Register i of tile t holds query q0 + t*32 + (i&8)*2 + 8hf + (i&7).
    auto half_s = [&](int it, const unsigned char* qa, const unsigned char* st) __attribute__((always_inline)) {
      const int q0 = stage_q0(it);
      carry = stage_live(q0);
      if (!carry) return;
      const bool need_mask = wave_k_first + 31 > bwd_key_hi<GENERAL>(g, q0) ||
                             (GENERAL && wave_k_first < bwd_key_lo<GENERAL>(g, q0 + BQS - 1));
      f32x16 s[QT];
#pragma unroll
      for (int t = 0; t < QT; ++t) s[t] = f32x16{};
      __builtin_amdgcn_s_setprio(1);              // its products first: the softmax waits on them
      stream(IQT{}, IKSD{}, IKSD{}, I1{}, s, qa, kvf);
      __builtin_amdgcn_s_setprio(0);
      auto softmax = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < QT; ++t)
#pragma unroll
          for (int gg = 0; gg < 2; ++gg) {
            const int qoff = t * 32 + 16 * gg + 8 * hf;
            float l8[8], pv[8];
            stat8(st, 0, qoff, l8);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              float p = fast_exp2(fmaf(s[t][8 * gg + e], g.scale_log2e, -l8[e]));
              if constexpr (decltype(masked)::value) {
                const int qq = q0 + qoff + e;
                if (GENERAL ? (kpos > bwd_key_hi<true>(g, qq) || kpos < bwd_key_lo<true>(g, qq))
                            : (g.causal && kpos > qq))
                  p = 0.f;
              }
              pv[e] = p;
            }
            pf[2 * t + gg] = O::from_f32(pv);
          }
      };
      if (need_mask) softmax(BoolTag<true>{});
      else softmax(BoolTag<false>{});
#pragma unroll
      for (int kk = 0; kk < QK; ++kk) *reinterpret_cast<F*>(px + (kg * QK + kk) * FB + lane * 16) = pf[kk];
    };
    // second half, P wave: dV^T += dO^T P
    auto half_dv = [&](const unsigned char* dt) __attribute__((always_inline)) {
      if (!carry) return;
      stream(IDT{}, IQK{}, IQK{}, I1{}, acc, dt, pf);
    };
    // second half, dS wave: dP = dO V^T, dS = P (dP - D) -> dsf
    auto half_dp = [&](int it, const unsigned char* da, const unsigned char* st) __attribute__((always_inline)) {
      carry = stage_live(stage_q0(it));
      if (!carry) return;
      // the accumulators start from -D of their rows: dP - D comes out of the products
      f32x16 dp[QT];
#pragma unroll
      for (int t = 0; t < QT; ++t)
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
          float d8[8];
          stat8(st, 1, t * 32 + 16 * gg + 8 * hf, d8);
#pragma unroll
          for (int e = 0; e < 8; ++e) dp[t][8 * gg + e] = d8[e];
        }
      __builtin_amdgcn_s_setprio(1);              // its products first: dS waits on them
      stream(IQT{}, IKSD{}, IKSD{}, I1{}, dp, da, kvf);
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int t = 0; t < QT; ++t)
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
          const F p8 = *reinterpret_cast<const F*>(px + (kg * QK + 2 * t + gg) * FB + lane * 16);
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = (float)p8[e] * dp[t][8 * gg + e];
          dsf[2 * t + gg] = O::from_f32(v);
        }
    };
    // first half, dS wave: dK^T += Q^T dS of the previous stage
    auto half_dk = [&](const unsigned char* qt) __attribute__((always_inline)) {
      if (!carry) return;
      stream(IDT{}, IQK{}, IQK{}, I1{}, acc, qt, dsf);
    };
    // middle barrier: P's LDS stores complete, no copy waited for
    auto half_barrier = []() __attribute__((always_inline)) {
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };

    // Step j (0..n_it) works on stage j, whose operands are in the parity-(j&1)
    // buffers (Q^T of stage j-1 in qt[(j-1)&1]); stage j+1's copies go to the other
    // parity, its Q^T at the middle barrier, once the dS waves are done with stage
    // j-1's. Unrolled by two so that every buffer is chosen at compile time. Each role
    // runs its own copy of the loop; both execute the same sequence of barriers.
    if (n_it > 0) {
      issue_step(0, qa0, da0, dt0, st0);
      issue_cols(0, g.qT, qt0);
    }
    for (int it = 0; it <= n_it && n_it > 0; it += 2) {
      wait_vmem();
      __syncthreads();
      if (it + 1 < n_it) issue_step(it + 1, qa1, da1, dt1, st1);
      if constexpr (PW) {
        if (it < n_it) half_s(it, qa0, st0);
      } else {
        half_dk(qt1);
      }
      half_barrier();
      if (it + 1 < n_it) issue_cols(it + 1, g.qT, qt1);
      if (it < n_it) {
        if constexpr (PW) half_dv(dt0);
        else half_dp(it, da0, st0);
      }
      if (it + 1 > n_it) break;
      wait_vmem();
      __syncthreads();
      if (it + 2 < n_it) issue_step(it + 2, qa0, da0, dt0, st0);
      if constexpr (PW) {
        if (it + 1 < n_it) half_s(it + 1, qa1, st1);
      } else {
        half_dk(qt0);
      }
      half_barrier();
      if (it + 2 < n_it) issue_cols(it + 2, g.qT, qt0);
      if (it + 1 < n_it) {
        if constexpr (PW) half_dv(dt1);
        else half_dp(it + 1, da1, st1);
      }
    }
    // register group gg of feature tile t holds features t*32 + 16gg + 8hf + [0, 8)
    if (kpos < N) {
      float* out = (PW ? g.dv : g.dk) + ((size_t)b * N + kpos) * dkv + (size_t)gk * DK;
      const float sc = PW ? 1.f : g.scale;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = acc[t][8 * gg + e] * sc;
          store8_f32(out + t * 32 + 16 * gg + 8 * hf, v);
        }
    }
  };
  if (pwave) run(BoolTag<true>{});
  else run(BoolTag<false>{});
}

}  // namespace bpt
