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
#include "bpt_device.hpp"
#include "bpt_launch.hpp"

namespace bpt {

// Rescale the running state only when a row maximum grows by more than 2^8 (in
// the exp2 domain): exp2(s - m) then stays below 256, exact enough in fp32 and
// bf16, and most key/value blocks need no rescale of o at all.
constexpr float kRescaleSlack = 8.0f;

template <typename T, int DK, int BQ, int BKV>
__global__ __launch_bounds__(BQ * 2, (4 * BKV * DK * (int)sizeof(T) <= 65536) ? 2 : 1) void
attention_kernel(T* QP, const T* __restrict__ KP, const T* __restrict__ VP, int N, int Np, int H,
                 int d, int causal, float scale_log2e, int n_qblocks, int n_items) {
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
  constexpr int STAGE = (KFR + VFR) * FB;
  constexpr int NCOPY = (KFR + VFR) * PCS;     // 1 KB copies per block
  constexpr int CPW = NCOPY / NW;
  static_assert(NCOPY % NW == 0, "copies per wave");
  __shared__ __align__(16) unsigned char lds0[STAGE];
  __shared__ __align__(16) unsigned char lds1[STAGE];

  // work item: XCD-aware (dispatch is round-robin over 8 XCDs), so one XCD walks
  // consecutive items: all query blocks of a (sequence, head), longest first.
  int item = blockIdx.x;
  if ((n_items & 7) == 0) item = (blockIdx.x & 7) * (n_items >> 3) + (blockIdx.x >> 3);
  const int bh = item / n_qblocks;
  const int qb = n_qblocks - 1 - (item - bh * n_qblocks);
  const int bi = bh / H, head = bh - bi * H;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rho = lane & 31, hf = lane >> 5;
  const int q0 = qb * BQ;
  const int qpos = q0 + wave * 32 + rho;       // this lane's query position
  const int wave_q_first = q0 + wave * 32;

  // this wave's Q fragments (B operand): packed row tile, the head's k-steps
  T* qfrag = QP + ((size_t)((bi * Np + wave_q_first) >> 5) * (d / 16) + head * KSD) * kFragElems;
  F qf[KSD];
#pragma unroll
  for (int kk = 0; kk < KSD; ++kk) qf[kk] = ld_packed(qfrag + kk * kFragElems, lane);

  const int n_kv = (N + BKV - 1) / BKV;
  const int q_last = min(q0 + BQ, N) - 1;
  const int kv_end = causal ? (q_last / BKV + 1) : n_kv;

  const T* kbase = KP + (size_t)bh * (Np / 32) * KSD * kFragElems;
  const T* vbase = VP + (size_t)bh * DT * (Np / 16) * kFragElems;

  // copy key/value block kb into an LDS stage (K fragments, then V fragments)
  auto issue = [&](int kb, unsigned char* buf) {
    const int kv0 = kb * BKV;
#pragma unroll
    for (int q = 0; q < CPW; ++q) {
      const int idx = wave * CPW + q;
      const int piece = idx % PCS, f = idx / PCS;
      const T* src;
      if (f < KFR) {
        src = kbase + ((size_t)(kv0 / 32) * KSD + f) * kFragElems;
      } else {
        const int ff = f - KFR, dt = ff / KK, kk = ff - dt * KK;
        src = vbase + ((size_t)dt * (Np / 16) + kv0 / 16 + kk) * kFragElems;
      }
      dma16(src + piece * (kFragElems / PCS) + lane * (8 / PCS), buf + f * FB + piece * 1024);
    }
  };

  f32x16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;   // m_run in the exp2 domain (scores * scale_log2e)

  auto block = [&](int kb, const unsigned char* buf) {
    const int kv0 = kb * BKV;
    // a wave whose 32 rows all precede this block has nothing to add
    if (causal && kv0 > wave_q_first + 31) return;
    f32x16 s[KT];
#pragma unroll
    for (int t = 0; t < KT; ++t) s[t] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KSD; ++kk)
#pragma unroll
      for (int t = 0; t < KT; ++t)
        O::mma(s[t], ld_packed(reinterpret_cast<const T*>(buf + (t * KSD + kk) * FB), lane), qf[kk]);
    // mask future keys and keys past the end (only blocks that can contain them)
    if ((kv0 + BKV > N) || (causal && kv0 + BKV - 1 > wave_q_first)) {
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kp = kv0 + t * 32 + c_row_pi(i, hf);
          if (kp >= N || (causal && kp > qpos)) s[t][i] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[t][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * scale_log2e;
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
    float lsum = 0.f;
    F pf[KK];
#pragma unroll
    for (int t = 0; t < KT; ++t) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float pe = fast_exp2(fmaf(s[t][8 * g + e], scale_log2e, -m_run));
          if constexpr (sizeof(T) == 2) pe = bf16_round(pe);
          p[e] = pe;
          lsum += pe;
        }
        pf[2 * t + g] = O::from_f32(p);
      }
    }
    l_run += lsum;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int t = 0; t < DT; ++t)
        O::mma(oacc[t], ld_packed(reinterpret_cast<const T*>(buf + (KFR + t * KK + kk) * FB), lane),
               pf[kk]);
  };

  // two static stages alternate; kv_end may be odd
  issue(0, lds0);
  for (int kb = 0; kb < kv_end; kb += 2) {
    wait_vmem();
    __syncthreads();             // stage 0 landed for every wave; stage 1 is free
    if (kb + 1 < kv_end) issue(kb + 1, lds1);
    block(kb, lds0);
    if (kb + 1 < kv_end) {
      wait_vmem();
      __syncthreads();           // stage 1 landed; stage 0 is free
      if (kb + 2 < kv_end) issue(kb + 2, lds0);
      block(kb + 1, lds1);
    }
  }

  // O = o / l, written in place over this wave's Q fragments (B-fragment order):
  // register group g of feature tile t holds features t*32 + 16g + 8hf + [0, 8).
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
#pragma unroll
  for (int t = 0; t < DT; ++t) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = oacc[t][8 * g + e] * inv;
      st_packed(qfrag + (2 * t + g) * kFragElems, 32 * hf + rho, v);
    }
  }
}

namespace {

template <typename T, int DK, int BQ, int BKV>
int run_attn(const LayerLaunch& L, hipStream_t s, char* err, size_t n) {
  const int nqb = (L.seq_len + BQ - 1) / BQ;
  const int items = L.batch * L.n_heads * nqb;
  const float scale = 1.4426950408889634f / sqrtf((float)DK);
  hipLaunchKernelGGL((attention_kernel<T, DK, BQ, BKV>), dim3(items), dim3(BQ * 2), 0, s,
                     (T*)L.q, (const T*)L.k, (const T*)L.vt, L.seq_len, L.seq_pad, L.n_heads,
                     L.d_model, L.causal, scale, nqb, items);
  return check_launch("attention", err, n);
}

template <typename T>
int dispatch_attn(const LayerLaunch& L, hipStream_t s, char* err, size_t n) {
  const int dk = L.d_head, bq = L.block_q, bkv = L.block_kv;
#define BPT_ATTN(DK_, BQ_, BKV_) \
  if (dk == DK_ && bq == BQ_ && bkv == BKV_) return run_attn<T, DK_, BQ_, BKV_>(L, s, err, n);
  BPT_ATTN(64, 64, 64)
  BPT_ATTN(64, 64, 128)
  BPT_ATTN(64, 128, 64)
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
