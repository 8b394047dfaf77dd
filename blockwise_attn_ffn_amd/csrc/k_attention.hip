// Attention of the BPT layer (gfx950): per (sequence, head, query block), the
// inner loop over key/value blocks with the running online-softmax state.
//
// "Blockwise Parallel Transformer — BPT" (aicassindra.com), section "The fused
// blockwise algorithm" (inner loop: s, m', alpha, l, o) and "Pitfalls and
// misconceptions" (key/value blocks after the query block are skipped, not
// computed and discarded). The running maximum and rescale are the ones of the
// FlashAttention paragraph of the transformer-cost page (raminaeye.github.io).
//
// Operands arrive as packed matrix-core fragments (bpt_device.hpp), written by the
// QKV projection; every sequence is padded to Np rows (a multiple of 128):
//   QP: B fragments over [packed rows, d]; the output O overwrites it in place.
//   KP: per (sequence, head) A fragments over [Np keys (pi order), d_k].
//   VP: per (sequence, head) A fragments over [d_k (pi order), Np keys].
// One workgroup = BQ query rows, one wave per 32 rows. S^T = K Q^T and
// O^T += V^T P^T on the matrix cores, so each lane owns one query row: row max and
// row sum are in-lane plus one exchange between the two lane halves. K and V
// blocks are copied global -> LDS by the LDS-DMA path into two static stages.
#include <type_traits>

#include "bpt_device.hpp"
#include "bpt_launch.hpp"

namespace bpt {

// Rescale the running state only when a row maximum grows by more than 2^8 (in
// the exp2 domain): exp2(s - m) then stays below 256, exact enough in fp32 and
// bf16, and most key/value blocks need no rescale of o at all.
constexpr float kRescaleSlack = 8.0f;
constexpr float kLn2 = 0.6931471805599453f;

// Maximum / sum of a value over the two lanes that hold the same query row
// (lanes l and l ^ 32): one lane-swap instruction, no LDS round trip.
__device__ inline float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Ring share: fold a finished row (o * inv, statistic lse_s, natural log) into the
// running state instead of writing it out. acc points at this wave's first output
// fragment in the fp32 copy of Q's fragment layout; lane holds 8 features of each
// of the 2 DT fragments. The state's statistic is read by both lane halves of the
// row before the lower half writes it back. A row's first merge (lse_acc = -inf)
// ignores whatever acc held.
//   lse = ln(e^la + e^ls),  O = e^(la - lse) O_acc + e^(ls - lse) o / l
template <int DT>
__device__ inline void merge_row(float* acc, int lane, const f32x16 (&oacc)[DT], float inv, float lse_s,
                                 float* lse_row, bool real_row, bool writer) {
  const float la = real_row ? *lse_row : -INFINITY;
  const float mx = fmaxf(la, lse_s);
  const float lse = mx + logf(expf(la - mx) + expf(lse_s - mx));
  const float wa = expf(la - lse), wb = expf(lse_s - lse) * inv;
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      float* p = acc + (size_t)(2 * t + g) * kFragElems + lane * 8;
      float a[8];
      if (wa != 0.f) load8_f32(p, a);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = oacc[t][8 * g + e] * wb;
        a[e] = wa != 0.f ? fmaf(wa, a[e], v) : v;
      }
      store8_f32(p, a);
    }
  if (writer && real_row) *lse_row = lse;
}

// Workgroups per CU the one-group kernel is built for: 2 when its two LDS stages
// fit 64 KB, else 1; bf16 at d_k 64 with 64-key tiles (32 KB of stages) runs 3,
// which leaves each wave 170 VGPRs and gives every SIMD a third wave to overlap
// one wave's softmax with another's products (measured 10% faster than 2 at the
// 64 x 1024-token, 16-head shape).
template <typename T, int DK, int BKV, bool SPLIT>
constexpr int attn_wgs_per_cu() {
  if (sizeof(T) == 2 && DK == 64 && BKV == 64 && !SPLIT) return 3;
  return (4 * BKV * DK * (int)sizeof(T) * (SPLIT ? 2 : 1) <= 65536) ? 2 : 1;
}

// Persistent workgroups. The work is a list of units: a unit is one query block,
// or, with the causal mask, the pair of query blocks (nqb-1-p, p) so that every
// unit has the same number of key/value blocks. Units are numbered (sequence,
// head) major; the workgroups on one XCD (dispatch is round-robin over 8 XCDs)
// take a contiguous range of units, so the query blocks of a head run together
// and share its K and V in that XCD's L2. A workgroup walks its key/value blocks
// ("visits") across all of its units without draining the copy pipeline.
//
// SPLIT: every operand computed in fp32 is carried as a pair of bf16 values
// (hi = bf16(v), lo = bf16(v - hi)), so that products keep ~16 significant bits:
// S = Qhi Khi + Qhi Klo + Qlo Khi and O += Vhi Phi + Vlo Phi + Vhi Plo; O is written
// as such a pair too. The LDS stage holds the hi fragments, then the lo ones.
template <typename T, int DK, int BQ, int BKV, bool SPLIT = false, bool MASKED = false, bool MERGE = false>
__global__ __launch_bounds__(BQ * 2, (attn_wgs_per_cu<T, DK, BKV, SPLIT>())) void
attention_kernel(T* QP, const T* __restrict__ KP, const T* __restrict__ VP, T* QPlo,
                 const T* __restrict__ KPlo, const T* __restrict__ VPlo, int N, int Np, int H,
                 int G, int d, int causal, int window, int chunk, float scale_log2e, int nqb,
                 int n_bh, float* lse, float* o_acc, float* lse_acc) {
  using O = Op<T>;
  using F = typename O::frag;
  constexpr int NW = BQ / 32;
  constexpr int PCS = frag_pieces<T>();
  constexpr int FB = 1024 * PCS;               // bytes per fragment
  constexpr int KSD = DK / 16;                 // k-steps over d_k
  constexpr int KT = BKV / 32;                 // key tiles per block (S^T tiles)
  constexpr int DT = DK / 32;                  // feature tiles (O^T tiles)
  constexpr int KK = BKV / 16;                 // key k-steps per block
  constexpr int KFR = KT * KSD, VFR = DT * KK; // fragments per block
  constexpr int HALF = (KFR + VFR) * FB;       // bytes of the hi (or lo) fragments
  constexpr int STAGE = HALF * (SPLIT ? 2 : 1);
  constexpr int NCOPY = (KFR + VFR) * PCS * (SPLIT ? 2 : 1);   // 1 KB copies per block
  constexpr int CPW = NCOPY / NW;
  // next unit's Q fetched during the last block of the current one (spare registers)
  constexpr bool kPrefetchQ = !SPLIT && DK * (int)sizeof(T) <= 128;
  // bf16: the block's K and V fragments are held in registers (64 VGPRs each)
  constexpr bool kPreload = sizeof(T) == 2 && !SPLIT;
  static_assert(NCOPY % NW == 0, "copies per wave");
  __shared__ __align__(16) unsigned char lds0[STAGE];
  __shared__ __align__(16) unsigned char lds1[STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rho = lane & 31, hf = lane >> 5;

  const int n_pairs = causal ? (nqb + 1) / 2 : nqb;
  const int n_units = n_bh * n_pairs;
  int part = 0, nparts = 1, j = blockIdx.x, M = gridDim.x;
  if ((gridDim.x & 7) == 0) {
    part = blockIdx.x & 7; nparts = 8; j = blockIdx.x >> 3; M = gridDim.x >> 3;
  }
  const int u_hi = (int)((long long)n_units * (part + 1) / nparts);

  // Visible keys of query position p (p past the end behaves as the last row):
  // causal: [0, p]; window w: [p - w + 1, p]; chunk C: up to the end of p's chunk.
  // MASKED instances (a window or chunk mask, or fewer key/value heads than query
  // heads) evaluate the general forms; the others compile to the plain causal /
  // unmasked bounds and read K and V of their own head.
  auto key_hi = [&](int p) {
    const int pc = min(p, N - 1);
    if (!causal) return N - 1;
    if constexpr (MASKED) return chunk ? min((pc / chunk + 1) * chunk, N) - 1 : pc;
    return pc;
  };
  auto key_lo = [&](int p) {
    if constexpr (MASKED) return window ? max(0, min(p, N - 1) - window + 1) : 0;
    return 0;
  };
  // query head h of sequence b reads key/value head h / (H / G) (grouped-query attention)
  // (MASKED instances only; the others have G == H)
  auto kv_head = [&](int bh) {
    const int bi = bh / H;
    return bi * G + (bh - bi * H) / (H / G);
  };
  // ---- visit cursor (wave-uniform): unit u, half w of it, query block qb,
  //      key/value block kb of kend, (sequence, head) bh
  // bh: (sequence, query head); kvh: (sequence, key/value head) of its K and V
  struct Cur { int u, w, qb, kb, kend, bh, kvh; };
  auto kvh_of = [&](const Cur& c) {
    if constexpr (MASKED) return c.kvh;
    return c.bh;
  };
  auto qblock = [&](int u, int w) {     // query block of half w of unit u, -1 if none
    const int p = u % n_pairs;
    if (!causal) return w == 0 ? p : -1;
    const int qa = nqb - 1 - p;
    return w == 0 ? qa : (p != qa ? p : -1);
  };
  auto start_qblock = [&](Cur& c) {
    c.qb = qblock(c.u, c.w);
    c.kb = key_lo(c.qb * BQ) / BKV;
    c.kend = key_hi(c.qb * BQ + BQ - 1) / BKV + 1;
    c.bh = c.u / n_pairs;
    c.kvh = MASKED ? kv_head(c.bh) : 0;   // unused by the plain instance
  };
  auto advance = [&](Cur& c) {          // c.u >= u_hi afterwards means: no more visits
    if (c.kb + 1 < c.kend) { ++c.kb; return; }
    if (c.w == 0 && qblock(c.u, 1) >= 0) c.w = 1;
    else { c.u += M; c.w = 0; }
    if (c.u < u_hi) start_qblock(c);
  };
  Cur cur;
  cur.u = (int)((long long)n_units * part / nparts) + j;
  cur.w = 0;
  if (cur.u >= u_hi) return;
  start_qblock(cur);

  auto qfrag_of = [&](const Cur& c) {   // this wave's Q fragments (B operand) of c's block
    const int bi = c.bh / H, head = c.bh - bi * H;
    return QP + ((size_t)((bi * Np + c.qb * BQ + wave * 32) >> 5) * (d / 16) + head * KSD) * kFragElems;
  };
  // copy key/value block c.kb of c.bh into an LDS stage (K fragments, then V
  // fragments; with SPLIT the lo fragments follow in the same order). Where every
  // wave's copies are of one kind (K or V, hi or lo; bf16), a wave takes one
  // branch per block and its copy sources are a base plus offsets that are
  // compile-time multiples of the fragment size and of one V row stride. Measured:
  // 10% faster with bf16 pairs, neutral at d_k 64; plain d_k 128 runs 9% faster
  // with the per-copy form below, whose longer copy section keeps the two
  // workgroups of a CU out of phase, and keeps it.
  constexpr bool kOneKind = sizeof(T) == 2 && (DK <= 64 || SPLIT) && CPW % (BKV / 16) == 0 &&
                            KFR % CPW == 0 && VFR % CPW == 0;
  const int f_first = wave * CPW;                          // first fragment slot of this wave
  const bool c_lo = SPLIT && f_first >= KFR + VFR;
  const int f_kind = c_lo ? f_first - (KFR + VFR) : f_first;   // slot within its half
  const bool c_k = f_kind < KFR;
  const uint32_t lane_off = (uint32_t)lane * 16u;
  auto issue = [&](const Cur& c, unsigned char* buf) __attribute__((always_inline)) {
    const int kv0 = c.kb * BKV;
    if constexpr (kOneKind) {
      unsigned char* dst = buf + f_first * FB;
      if (c_k) {
        const char* kb = reinterpret_cast<const char*>(
            (c_lo ? KPlo : KP) + ((size_t)kvh_of(c) * (Np / 32) + kv0 / 32) * KSD * kFragElems) +
            (size_t)f_kind * FB;
#pragma unroll
        for (int q = 0; q < CPW; ++q) dma16(kb + q * FB + lane_off, dst + q * FB);
      } else {
        // V fragment ff = f_kind - KFR + q: feature tile ff / KK, key step ff % KK
        const size_t S = (size_t)(Np / 16) * FB;          // bytes per feature tile
        const char* vb = reinterpret_cast<const char*>(
            (c_lo ? VPlo : VP) + ((size_t)kvh_of(c) * DT * (Np / 16) + kv0 / 16) * kFragElems) +
            (size_t)((f_kind - KFR) / KK) * S;
#pragma unroll
        for (int q = 0; q < CPW; ++q) dma16(vb + (q / KK) * S + (q % KK) * FB + lane_off, dst + q * FB);
      }
    } else {
      const size_t koff = (size_t)kvh_of(c) * (Np / 32) * KSD * kFragElems;
      const size_t voff = (size_t)kvh_of(c) * DT * (Np / 16) * kFragElems;
#pragma unroll
      for (int q = 0; q < CPW; ++q) {
        const int idx = wave * CPW + q;
        const int piece = idx % PCS, f2 = idx / PCS;
        const bool lo = SPLIT && f2 >= KFR + VFR;
        const int f = lo ? f2 - (KFR + VFR) : f2;
        const T* src;
        if (f < KFR) {
          src = (lo ? KPlo : KP) + koff + ((size_t)(kv0 / 32) * KSD + f) * kFragElems;
        } else {
          const int ff = f - KFR, dt = ff / KK, kk = ff - dt * KK;
          src = (lo ? VPlo : VP) + voff + ((size_t)dt * (Np / 16) + kv0 / 16 + kk) * kFragElems;
        }
        dma16(src + piece * (kFragElems / PCS) + lane * (8 / PCS), buf + f2 * FB + piece * 1024);
      }
    }
  };

  F qf[KSD], qn[KSD], ql[SPLIT ? KSD : 1];
  auto load_q = [&](const Cur& c, F (&dst)[KSD]) {
    const T* qp = qfrag_of(c);
#pragma unroll
    for (int kk = 0; kk < KSD; ++kk) dst[kk] = ld_packed(qp + kk * kFragElems, lane);
    if constexpr (SPLIT) {
      const T* qlp = QPlo + (qp - QP);
#pragma unroll
      for (int kk = 0; kk < KSD; ++kk) ql[kk] = ld_packed(qlp + kk * kFragElems, lane);
    }
  };
  f32x16 oacc[DT];
  float m_run, l_run;                   // m_run in the exp2 domain (scores * scale_log2e)
  auto reset = [&]() {
#pragma unroll
    for (int t = 0; t < DT; ++t) oacc[t] = f32x16{};
    m_run = -INFINITY;
    l_run = 0.f;
  };

  // one key/value block of the current query block; the last one also writes
  // O = o / l in place over this wave's Q fragments and resets the state
  auto visit = [&](const Cur& c, const Cur& nx, const unsigned char* buf) {
    const int kv0 = c.kb * BKV;
    const int wave_q_first = c.qb * BQ + wave * 32, qpos = wave_q_first + rho;
    const bool last = c.kb == c.kend - 1;
    if (kPrefetchQ && last && nx.u < u_hi) load_q(nx, qn);
    // a wave whose 32 rows see no key of this block has nothing to add
    if (kv0 <= key_hi(wave_q_first + 31) && (!MASKED || kv0 + BKV - 1 >= key_lo(wave_q_first))) {
      // bf16: all K fragments of the block are read from LDS first (one wait per
      // product instead of a round trip each); V's are issued right after the
      // S products, in flight during the softmax
      f32x16 s[KT];
#pragma unroll
      for (int t = 0; t < KT; ++t) s[t] = f32x16{};
      F kf[kPreload ? KFR : 1];
      if constexpr (kPreload) {
#pragma unroll
        for (int kk = 0; kk < KSD; ++kk)
#pragma unroll
          for (int t = 0; t < KT; ++t)
            kf[t * KSD + kk] = ld_packed(reinterpret_cast<const T*>(buf + (t * KSD + kk) * FB), lane);
        // d_k 64: every read in flight before the first product (measured faster);
        // d_k 128 runs faster with the reads interleaved among the products
        if constexpr (DK <= 64) __builtin_amdgcn_sched_barrier(0);
      }
      // d_k 128: this wave's products and softmax run at raised priority, so a wave
      // in its compute section is issued ahead of one copying or waiting at the
      // barrier (measured 7% faster at d_k 128; no gain at d_k 64 or with bf16 pairs)
      if constexpr (DK > 64 && !SPLIT) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kk = 0; kk < KSD; ++kk)
#pragma unroll
        for (int t = 0; t < KT; ++t) {
          if constexpr (kPreload) {
            O::mma(s[t], kf[t * KSD + kk], qf[kk]);
          } else {
            const F kh = ld_packed(reinterpret_cast<const T*>(buf + (t * KSD + kk) * FB), lane);
            O::mma(s[t], kh, qf[kk]);
            if constexpr (SPLIT) {
              O::mma(s[t], ld_packed(reinterpret_cast<const T*>(buf + HALF + (t * KSD + kk) * FB), lane),
                     qf[kk]);
              O::mma(s[t], kh, ql[kk]);
            }
          }
        }
      F vf[kPreload ? VFR : 1];
      if constexpr (kPreload) {
#pragma unroll
        for (int f = 0; f < VFR; ++f)
          vf[f] = ld_packed(reinterpret_cast<const T*>(buf + (KFR + f) * FB), lane);
        __builtin_amdgcn_sched_barrier(0);
      }
      // mask future keys and keys past the end (only blocks that can contain them):
      // register i of tile t holds key kv0 + t*32 + (i&8)*2 + 8hf + (i&7)
      if (kv0 + BKV - 1 > key_hi(wave_q_first) || (MASKED && kv0 < key_lo(wave_q_first + 31))) {
        const int lim = key_hi(qpos) - kv0 - 8 * hf, lim_lo = key_lo(qpos) - kv0 - 8 * hf;
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int off = t * 32 + (i & 8) * 2 + (i & 7);
            if (off > lim || (MASKED && off < lim_lo)) s[t][i] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[t][i]);
      mx = pair_max(mx) * scale_log2e;
      // lazy rescale: only when some row's maximum grew past the slack
      if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleSlack) != 0) {
        const float m_new = fmaxf(m_run, mx);
        // 0 on a row's first visit (m_run = -inf); 1 if the row has seen no key yet
        const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int t = 0; t < DT; ++t) oacc[t] *= alpha;
      }
      // p = exp2(s * scale - m); l sums p in fp32, P feeds the product in T. A row
      // that has seen no key yet (a window's first blocks) has m = -inf: shift 0
      const float m_use = (MASKED && m_run == -INFINITY) ? 0.f : m_run;
      float lsum = 0.f;
      F pf[KK], pl[SPLIT ? KK : 1];
#pragma unroll
      for (int t = 0; t < KT; ++t) {
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          float p[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            p[e] = fast_exp2(fmaf(s[t][8 * g + e], scale_log2e, -m_use));
            lsum += p[e];
          }
          pf[2 * t + g] = O::from_f32(p);
          if constexpr (SPLIT) {
            float r[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) r[e] = p[e] - bf16_round(p[e]);
            pl[2 * t + g] = O::from_f32(r);
          }
        }
      }
      l_run += lsum;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          if constexpr (kPreload) {
            O::mma(oacc[t], vf[t * KK + kk], pf[kk]);
          } else {
            const F vh = ld_packed(reinterpret_cast<const T*>(buf + (KFR + t * KK + kk) * FB), lane);
            O::mma(oacc[t], vh, pf[kk]);
            if constexpr (SPLIT) {
              O::mma(oacc[t],
                     ld_packed(reinterpret_cast<const T*>(buf + HALF + (KFR + t * KK + kk) * FB), lane),
                     pf[kk]);
              O::mma(oacc[t], vh, pl[kk]);
            }
          }
        }
      if constexpr (DK > 64 && !SPLIT) __builtin_amdgcn_s_setprio(0);
    }
    if (last) {
      // register group g of feature tile t holds features t*32 + 16g + 8hf + [0, 8)
      T* qp = qfrag_of(c);
      const float l_tot = pair_sum(l_run);
      const float inv = 1.0f / l_tot;
      // saved statistic of the row: l_tot sums exp2(s * scale_log2e - m_run), so the
      // softmax normaliser of the scaled scores is exp(ln2 (m_run + log2 l_tot))
      if (lse != nullptr && hf == 0 && qpos < N)
        lse[(size_t)c.bh * N + qpos] = (m_run + log2f(l_tot)) * kLn2;
      // the ring share's merge (instances for bf16 operands only: fp32 fragments
      // have two pieces)
      if constexpr (MERGE && sizeof(T) == 2 && !SPLIT) {
        merge_row<DT>(o_acc + (qp - QP), lane, oacc, inv, (m_run + log2f(l_tot)) * kLn2,
                      lse_acc + (size_t)c.bh * N + min(qpos, N - 1), qpos < N, hf == 0);
      } else {
#pragma unroll
        for (int t = 0; t < DT; ++t) {
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = oacc[t][8 * g + e] * inv;
            st_packed(qp + (2 * t + g) * kFragElems, lane, v);
            if constexpr (SPLIT) {
#pragma unroll
              for (int e = 0; e < 8; ++e) v[e] -= bf16_round(v[e]);
              st_packed(QPlo + (qp - QP) + (2 * t + g) * kFragElems, lane, v);
            }
          }
        }
      }
      reset();
      if (nx.u < u_hi) {
        if constexpr (kPrefetchQ) {
#pragma unroll
          for (int kk = 0; kk < KSD; ++kk) qf[kk] = qn[kk];
        } else {
          load_q(nx, qf);
        }
      }
    }
  };

  // two static stages alternate; visit v uses stage v % 2
  reset();
  load_q(cur, qf);
  issue(cur, lds0);
  Cur nxt = cur;
  advance(nxt);
  for (;;) {
    wait_vmem();
    __syncthreads();             // stage 0 landed for every wave; stage 1 is free
    if (nxt.u < u_hi) issue(nxt, lds1);
    visit(cur, nxt, lds0);
    if (nxt.u >= u_hi) break;
    cur = nxt;
    advance(nxt);
    wait_vmem();
    __syncthreads();             // stage 1 landed; stage 0 is free
    if (nxt.u < u_hi) issue(nxt, lds0);
    visit(cur, nxt, lds1);
    if (nxt.u >= u_hi) break;
    cur = nxt;
    advance(nxt);
  }
}

// ---------------------------------------------------------------------------
// Two-group schedule (bf16, d_k 128, query blocks of 128 rows). One workgroup of
// 8 waves per CU takes a pair of adjacent query blocks ("super-block") that share
// one key/value stream: group 0 (waves 0-3) the even block, group 1 (waves 4-7)
// the odd one, 32 query rows per wave as above. The two groups run half a step
// apart: while one group multiplies (P V of the previous key/value block, then S
// of the current one), the other runs the softmax of its scores, so each SIMD,
// which holds one wave of each group, has matrix-core and vector work in flight
// together. K and V have two LDS buffers each; at the start of step k group 0
// copies K of visit k+1 and group 1 copies V of visit k, and both land before
// step k+1, when they are first read. Work units are pairs of super-blocks
// (S-1-p, p) with the causal mask, as for the one-group kernel.
// ---------------------------------------------------------------------------
template <int DK, int BKV, bool MASKED = false, bool MERGE = false>
__global__ __launch_bounds__(512, 1) void attention_pair_kernel(
    bf16* QP, const bf16* __restrict__ KP, const bf16* __restrict__ VP, int N, int Np, int H,
    int G, int d, int causal, int window, int chunk, float scale_log2e, int nqb, int n_bh,
    float* lse, float* o_acc, float* lse_acc) {
  using O = Op<bf16>;
  using F = O::frag;
  constexpr int BQ = 128, NWG = 4, FB = 1024;
  constexpr int KSD = DK / 16;                 // k-steps over d_k
  constexpr int KT = BKV / 32;                 // key tiles per block (S^T tiles)
  constexpr int DT = DK / 32;                  // feature tiles (O^T tiles)
  constexpr int KK = BKV / 16;                 // key k-steps per block
  constexpr int KFR = KT * KSD, VFR = DT * KK; // fragments per block
  constexpr int KCPW = KFR / NWG;              // K copies per group-0 wave
  constexpr int VCPW = VFR / NWG;              // V copies per group-1 wave
  static_assert(KFR % NWG == 0 && VFR % NWG == 0 && VCPW <= KK && KK % VCPW == 0,
                "a group-1 wave copies consecutive key steps of one feature tile of V");
  __shared__ __align__(16) unsigned char kbuf[2][KFR * FB];
  __shared__ __align__(16) unsigned char vbuf[2][VFR * FB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, wq = wave & 3;
  const int rho = lane & 31, hf = lane >> 5;
  const uint32_t lane_off = (uint32_t)lane * 16u;

  const int nsb = (nqb + 1) / 2;               // super-blocks
  const int n_pairs = causal ? (nsb + 1) / 2 : nsb;
  const int n_units = n_bh * n_pairs;
  int part = 0, nparts = 1, j = blockIdx.x, M = gridDim.x;
  if ((gridDim.x & 7) == 0) {
    part = blockIdx.x & 7; nparts = 8; j = blockIdx.x >> 3; M = gridDim.x >> 3;
  }
  const int u_hi = (int)((long long)n_units * (part + 1) / nparts);

  // Visible keys of query position p (p past the end behaves as the last row):
  // causal: [0, p]; window w: [p - w + 1, p]; chunk C: up to the end of p's chunk.
  // MASKED instances (a window or chunk mask, or fewer key/value heads than query
  // heads) evaluate the general forms; the others compile to the plain causal /
  // unmasked bounds and read K and V of their own head.
  auto key_hi = [&](int p) {
    const int pc = min(p, N - 1);
    if (!causal) return N - 1;
    if constexpr (MASKED) return chunk ? min((pc / chunk + 1) * chunk, N) - 1 : pc;
    return pc;
  };
  auto key_lo = [&](int p) {
    if constexpr (MASKED) return window ? max(0, min(p, N - 1) - window + 1) : 0;
    return 0;
  };
  // query head h of sequence b reads key/value head h / (H / G) (grouped-query attention)
  // (MASKED instances only; the others have G == H)
  auto kv_head = [&](int bh) {
    const int bi = bh / H;
    return bi * G + (bh - bi * H) / (H / G);
  };
  // visit cursor over super-blocks (wave-uniform), as in the one-group kernel
  struct Cur { int u, w, sb, kb, kend, bh, kvh; };
  auto kvh_of = [&](const Cur& c) {
    if constexpr (MASKED) return c.kvh;
    return c.bh;
  };
  auto sblock = [&](int u, int w) {
    const int p = u % n_pairs;
    if (!causal) return w == 0 ? p : -1;
    const int qa = nsb - 1 - p;
    return w == 0 ? qa : (p != qa ? p : -1);
  };
  auto start_half = [&](Cur& c) {
    c.sb = sblock(c.u, c.w);
    c.kb = key_lo(c.sb * 2 * BQ) / BKV;
    c.kend = key_hi(c.sb * 2 * BQ + 2 * BQ - 1) / BKV + 1;
    c.bh = c.u / n_pairs;
    c.kvh = MASKED ? kv_head(c.bh) : 0;   // unused by the plain instance
  };
  auto advance = [&](Cur& c) {          // c.u >= u_hi afterwards: no more visits
    if (c.kb + 1 < c.kend) { ++c.kb; return; }
    if (c.w == 0 && sblock(c.u, 1) >= 0) c.w = 1;
    else { c.u += M; c.w = 0; }
    if (c.u < u_hi) start_half(c);
  };
  Cur ck;
  ck.u = (int)((long long)n_units * part / nparts) + j;
  ck.w = 0;
  if (ck.u >= u_hi) return;
  start_half(ck);

  // this wave's query block in visit c's super-block (-1 if the block is past the end)
  auto my_qb = [&](const Cur& c) { const int qb = 2 * c.sb + grp; return qb < nqb ? qb : -1; };
  auto qfrag_of = [&](const Cur& c, int qb) {
    const int bi = c.bh / H, head = c.bh - bi * H;
    return QP + ((size_t)((bi * Np + qb * BQ + wq * 32) >> 5) * (d / 16) + head * KSD) * kFragElems;
  };
  F qf[KSD];
  auto load_q = [&](const Cur& c) __attribute__((always_inline)) {
    const int qb = my_qb(c);
    if (qb < 0) return;
    const bf16* qp = qfrag_of(c, qb);
#pragma unroll
    for (int kk = 0; kk < KSD; ++kk) qf[kk] = ld_packed(qp + kk * kFragElems, lane);
  };
  // group 0 copies visit c's K block, group 1 its V block (VCPW consecutive key
  // steps of one feature tile per wave)
  auto issue_k = [&](const Cur& c, unsigned char* buf) __attribute__((always_inline)) {
    const char* src = reinterpret_cast<const char*>(
        KP + (((size_t)kvh_of(c) * (Np / 32) + c.kb * BKV / 32) * KSD + wq * KCPW) * kFragElems);
#pragma unroll
    for (int q = 0; q < KCPW; ++q) dma16(src + q * FB + lane_off, buf + (wq * KCPW + q) * FB);
  };
  auto issue_v = [&](const Cur& c, unsigned char* buf) __attribute__((always_inline)) {
    const int dt = wq * VCPW / KK, kk0 = wq * VCPW % KK;
    const char* src = reinterpret_cast<const char*>(
        VP + (((size_t)kvh_of(c) * DT + dt) * (Np / 16) + c.kb * BKV / 16 + kk0) * kFragElems);
#pragma unroll
    for (int q = 0; q < VCPW; ++q) dma16(src + q * FB + lane_off, buf + (wq * VCPW + q) * FB);
  };

  f32x16 oacc[DT], s[KT];
  F pf[KK];
  float m_run = -INFINITY, l_run = 0.f;
  bool s_valid = false, p_valid = false;
  auto reset = [&]() {
#pragma unroll
    for (int t = 0; t < DT; ++t) oacc[t] = f32x16{};
    m_run = -INFINITY;
    l_run = 0.f;
  };
  reset();

  // product step of visit k: P V of the previous visit (V in vb), O of the previous
  // half when that visit was its last, then S of visit k (K in kb)
  auto mstep = [&](const Cur& cp, bool has_p, const Cur& c, bool has_c, const unsigned char* kb,
                   const unsigned char* vb) __attribute__((always_inline)) {
    // the multiplying wave of a SIMD is issued ahead of the one in its softmax
    // (measured 6% faster than equal priorities)
    __builtin_amdgcn_s_setprio(1);
    if (p_valid) {
      // V fragments of key step kk+1 are read while the products of kk run
      F va[2][DT];
      auto ldv = [&](int kk, F (&dst)[DT]) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < DT; ++t)
          dst[t] = ld_packed(reinterpret_cast<const bf16*>(vb + (t * KK + kk) * FB), lane);
      };
      ldv(0, va[0]);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        if (kk + 1 < KK) ldv(kk + 1, va[(kk + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < DT; ++t) O::mma(oacc[t], va[kk & 1][t], pf[kk]);
        __builtin_amdgcn_sched_barrier(0);
      }
      p_valid = false;
    }
    if (has_p && cp.kb == cp.kend - 1) {
      const int qb = my_qb(cp);
      if (qb >= 0) {
        // register group g of feature tile t holds features t*32 + 16g + 8hf + [0, 8)
        bf16* qp = qfrag_of(cp, qb);
        const float l_tot = pair_sum(l_run);
        const float inv = 1.0f / l_tot;
        const int qpos = qb * BQ + wq * 32 + rho;
        if (lse != nullptr && hf == 0 && qpos < N)
          lse[(size_t)cp.bh * N + qpos] = (m_run + log2f(l_tot)) * kLn2;
        if constexpr (MERGE) {
          merge_row<DT>(o_acc + (qp - QP), lane, oacc, inv, (m_run + log2f(l_tot)) * kLn2,
                        lse_acc + (size_t)cp.bh * N + min(qpos, N - 1), qpos < N, hf == 0);
        } else {
#pragma unroll
          for (int t = 0; t < DT; ++t) {
#pragma unroll
            for (int g = 0; g < 2; ++g) {
              float v[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) v[e] = oacc[t][8 * g + e] * inv;
              st_packed(qp + (2 * t + g) * kFragElems, lane, v);
            }
          }
        }
      }
      reset();
    }
    s_valid = false;
    if (has_c) {
      const int qb = my_qb(c);
      const int wave_q_first = qb * BQ + wq * 32;
      // a wave whose 32 rows see no key of this block has nothing to add
      if (qb >= 0 && c.kb * BKV <= key_hi(wave_q_first + 31) &&
          (!MASKED || c.kb * BKV + BKV - 1 >= key_lo(wave_q_first))) {
#pragma unroll
        for (int t = 0; t < KT; ++t) s[t] = f32x16{};
        // K fragments of k-step kk+1 are read while the products of kk run
        F ka[2][KT];
        auto ldk = [&](int kk, F (&dst)[KT]) __attribute__((always_inline)) {
#pragma unroll
          for (int t = 0; t < KT; ++t)
            dst[t] = ld_packed(reinterpret_cast<const bf16*>(kb + (t * KSD + kk) * FB), lane);
        };
        ldk(0, ka[0]);
#pragma unroll
        for (int kk = 0; kk < KSD; ++kk) {
          if (kk + 1 < KSD) ldk(kk + 1, ka[(kk + 1) & 1]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int t = 0; t < KT; ++t) O::mma(s[t], ka[kk & 1][t], qf[kk]);
          __builtin_amdgcn_sched_barrier(0);
        }
        s_valid = true;
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // softmax step of visit c: mask, running maximum (lazy rescale), P and l
  auto vstep = [&](const Cur& c) __attribute__((always_inline)) {
    if (!s_valid) return;
    const int kv0 = c.kb * BKV;
    const int wave_q_first = my_qb(c) * BQ + wq * 32, qpos = wave_q_first + rho;
    // mask future keys and keys past the end (only blocks that can contain them):
    // register i of tile t holds key kv0 + t*32 + (i&8)*2 + 8hf + (i&7)
    if (kv0 + BKV - 1 > key_hi(wave_q_first) || (MASKED && kv0 < key_lo(wave_q_first + 31))) {
      const int lim = key_hi(qpos) - kv0 - 8 * hf, lim_lo = key_lo(qpos) - kv0 - 8 * hf;
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int off = t * 32 + (i & 8) * 2 + (i & 7);
          if (off > lim || (MASKED && off < lim_lo)) s[t][i] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[t][i]);
    mx = pair_max(mx) * scale_log2e;
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleSlack) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < DT; ++t) oacc[t] *= alpha;
    }
    const float m_use = (MASKED && m_run == -INFINITY) ? 0.f : m_run;   // no key seen yet
    float lsum = 0.f;
#pragma unroll
    for (int t = 0; t < KT; ++t) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = fast_exp2(fmaf(s[t][8 * g + e], scale_log2e, -m_use));
          lsum += p[e];
        }
        pf[2 * t + g] = O::from_f32(p);
      }
    }
    l_run += lsum;
    s_valid = false;
    p_valid = true;
  };

  // step k: [even half] group 0 multiplies for visit k, group 1 runs the softmax of
  // visit k-1; [odd half] group 0 the softmax of visit k, group 1 multiplies for k.
  // A final step with no visit k finishes P V and O of the last visit. Each group
  // runs its own copy of the loop (the phase order is a compile-time constant);
  // both execute the same sequence of barriers.
  auto run = [&](auto group) __attribute__((always_inline)) {
    constexpr int G = decltype(group)::value;
    load_q(ck);
    if constexpr (G == 0) issue_k(ck, kbuf[0]);
    Cur cp = ck;                     // visit k-1 (valid from k = 1)
    Cur cn = ck;                     // visit k+1
    advance(cn);
    for (int k = 0;; ++k) {
      const bool has_k = ck.u < u_hi, has_n = cn.u < u_hi, has_p = k > 0;
      wait_vmem();
      __syncthreads();               // K(k) and V(k-1) have landed
      // a new half starts at visit k: both groups are done with the old Q (their S
      // of visit k-1 ran in the previous step), so its Q is read now, ahead of the
      // copies (waiting for it does not wait for them)
      if (has_p && has_k && cp.kb == cp.kend - 1) load_q(ck);
      if constexpr (G == 0) {
        if (has_n) issue_k(cn, kbuf[(k + 1) & 1]);
        mstep(cp, has_p, ck, has_k, kbuf[k & 1], vbuf[(k + 1) & 1]);
      } else {
        if (has_k) issue_v(ck, vbuf[k & 1]);
        if (has_p) vstep(cp);
      }
      __builtin_amdgcn_s_barrier();  // half step: no copy is waited for here
      if constexpr (G == 0) {
        if (has_k) vstep(ck);
      } else {
        mstep(cp, has_p, ck, has_k, kbuf[k & 1], vbuf[(k + 1) & 1]);
      }
      if (!has_k) break;
      cp = ck;
      ck = cn;
      advance(cn);
    }
  };
  if (grp == 0) run(std::integral_constant<int, 0>{});
  else run(std::integral_constant<int, 1>{});
}

namespace {

// Compute units of the current device, queried on every call (a cheap attribute
// read; no cached state, so concurrent callers and several devices are safe).
int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  return cus;
}

template <typename T, int DK, int BQ, int BKV, bool SPLIT = false>
int run_attn(const LayerLaunch& L, hipStream_t s, char* err, size_t n) {
  const int nqb = (L.seq_len + BQ - 1) / BQ;
  const int n_bh = L.batch * L.n_heads;
  const int units = n_bh * (L.causal ? (nqb + 1) / 2 : nqb);
  // workgroups resident at once (attn_wgs_per_cu)
  constexpr int per_cu = attn_wgs_per_cu<T, DK, BKV, SPLIT>();
  int grid = device_cus() * per_cu;
  if (units < grid) grid = units;
  const float scale = 1.4426950408889634f / sqrtf((float)DK);
  // window / chunk masks and grouped key/value heads run the general instance;
  // plain causal or unmasked multi-head attention the other
  const bool general = L.window || L.chunk || L.n_kv_heads != L.n_heads;
  auto kern = general ? attention_kernel<T, DK, BQ, BKV, SPLIT, true>
                      : attention_kernel<T, DK, BQ, BKV, SPLIT, false>;
  if (L.o_acc != nullptr) {
    // the ring share's merging instance exists for the tiling it uses at d_k 64
    bool have = false;
    if constexpr (sizeof(T) == 2 && !SPLIT && DK == 64 && BQ == 128 && BKV == 64) {
      if (!general) {
        kern = attention_kernel<T, DK, BQ, BKV, SPLIT, false, true>;
        have = true;
      }
    }
    if (!have) {
      set_err(err, n, "attention: no merging instance for this shape%s", "");
      return 1;
    }
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(BQ * 2), 0, s,
                     (T*)L.q, (const T*)L.k, (const T*)L.vt, (T*)L.q_lo, (const T*)L.k_lo,
                     (const T*)L.vt_lo, L.seq_len, L.seq_pad, L.n_heads, L.n_kv_heads, L.d_model,
                     L.causal, L.window, L.chunk, scale, nqb, n_bh, L.lse, L.o_acc, L.lse_acc);
  return check_launch("attention", err, n);
}

template <int DK, int BKV>
int run_attn_pair(const LayerLaunch& L, hipStream_t s, char* err, size_t n) {
  const int nqb = (L.seq_len + 127) / 128;
  const int n_bh = L.batch * L.n_heads;
  const int nsb = (nqb + 1) / 2;
  const int units = n_bh * (L.causal ? (nsb + 1) / 2 : nsb);
  int grid = device_cus();
  if (units < grid) grid = units;
  const float scale = 1.4426950408889634f / sqrtf((float)DK);
  const bool general = L.window || L.chunk || L.n_kv_heads != L.n_heads;
  auto kern = general ? attention_pair_kernel<DK, BKV, true> : attention_pair_kernel<DK, BKV, false>;
  if (L.o_acc != nullptr) {
    // the ring share's merging instance exists for the tiling it uses at d_k 128
    bool have = false;
    if constexpr (DK == 128 && BKV == 64) {
      if (!general) {
        kern = attention_pair_kernel<DK, BKV, false, true>;
        have = true;
      }
    }
    if (!have) {
      set_err(err, n, "attention: no merging instance for this shape%s", "");
      return 1;
    }
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(512), 0, s, (bf16*)L.q,
                     (const bf16*)L.k, (const bf16*)L.vt, L.seq_len, L.seq_pad, L.n_heads,
                     L.n_kv_heads, L.d_model, L.causal, L.window, L.chunk, scale, nqb, n_bh, L.lse,
                     L.o_acc, L.lse_acc);
  return check_launch("attention", err, n);
}

template <typename T>
int dispatch_attn(const LayerLaunch& L, hipStream_t s, char* err, size_t n) {
  const int dk = L.d_head, bq = L.block_q, bkv = L.block_kv;
  if constexpr (sizeof(T) == 2) {
    // two-group schedule for d_k 128 only: at d_k 64 the softmax half step is
    // about twice the product half step and the one-group kernel measured faster
    if (!L.split && dk == 128 && bq == 128) {
      if (bkv == 64) return run_attn_pair<128, 64>(L, s, err, n);
      if (bkv == 128) return run_attn_pair<128, 128>(L, s, err, n);
    }

    if (L.split) {
      // pairs of fragments double the LDS stage: key/value tiles of 64 keys
      // (value-neutral: the online softmax is exact for any tiling)
      if (dk == 64 && bq == 64) return run_attn<T, 64, 64, 64, true>(L, s, err, n);
      if (dk == 64 && bq == 128) return run_attn<T, 64, 128, 64, true>(L, s, err, n);
      if (dk == 128 && bq == 64) return run_attn<T, 128, 64, 64, true>(L, s, err, n);
      if (dk == 128 && bq == 128) return run_attn<T, 128, 128, 64, true>(L, s, err, n);
    }
  }
#define BPT_ATTN(DK_, BQ_, BKV_) \
  if (dk == DK_ && bq == BQ_ && bkv == BKV_) return run_attn<T, DK_, BQ_, BKV_>(L, s, err, n);
  BPT_ATTN(64, 64, 64)
  BPT_ATTN(64, 64, 128)
  BPT_ATTN(64, 128, 64)
  // bf16 at d_k 64: key/value blocks of 128 run as two tiles of 64 (value-neutral:
  // the online softmax is exact for any tiling), at 3 workgroups per CU
  if (sizeof(T) == 2 && dk == 64 && bq == 128 && bkv == 128) return run_attn<T, 64, 128, 64>(L, s, err, n);
  BPT_ATTN(64, 128, 128)
  BPT_ATTN(128, 64, 64)
  BPT_ATTN(128, 128, 64)
  if constexpr (sizeof(T) == 2) {
    BPT_ATTN(128, 64, 128)
    BPT_ATTN(128, 128, 128)
  }
#undef BPT_ATTN
  set_err(err, n, "no attention kernel for this head size / block sizes%s", "");
  return 1;
}

}  // namespace

int launch_attention(const LayerLaunch& L, hipStream_t s, char* err, size_t n) {
  if (L.compute_f32) return dispatch_attn<float>(L, s, err, n);
  return dispatch_attn<bf16>(L, s, err, n);
}

}  // namespace bpt
