// Attention of the BPT layer (gfx950): per (sequence, head, query block), the
// inner loop over key/value blocks with the running online-softmax state.
//
// "Blockwise Parallel Transformer — BPT" (aicassindra.com), section "The fused
// blockwise algorithm" (inner loop: s, m', alpha, l, o) and "Pitfalls and
// misconceptions" (key/value blocks after the query block are skipped, not
// computed and discarded). The running maximum / rescale is the one described in
// the FlashAttention paragraph of the transformer-cost page (raminaeye.github.io).
#include "bpt_device.hpp"
#include "bpt_launch.hpp"

namespace bpt {

// ---------------------------------------------------------------------------
// Attention: one workgroup per (sequence, head, query block of BQ rows), one
// wave per 32 query rows. S^T = K Q^T and O^T += V^T P^T on the matrix cores,
// so each lane owns one query row: row max / row sum are in-lane plus one
// exchange between the two lane halves. K and V^T tiles are staged in LDS,
// double-buffered. Causal: key blocks past the query block are never visited.
// ---------------------------------------------------------------------------
template <typename T, int DK, int BQ, int BKV>
__global__ __launch_bounds__(BQ * 2, 2) void attention_kernel(
    const T* Qg, const T* __restrict__ Kg, const T* __restrict__ Vt, T* Og, int N,
    int H, int d, int ldv, int causal, float scale_log2e, int n_qblocks, int n_items) {
  using O = Op<T>;
  constexpr int NW = BQ / 32;
  constexpr int NTH = NW * 64;
  constexpr int KCPR = DK / 8, VCPR = BKV / 8;
  constexpr int KCH = BKV * KCPR / NTH, VCH = DK * VCPR / NTH;
  constexpr int ST = BKV / 32;    // S^T tiles (32 keys each)
  constexpr int DT = DK / 32;     // O^T tiles (32 features each)
  static_assert(KCH * NTH == BKV * KCPR && VCH * NTH == DK * VCPR, "staging split");

  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* Ks = reinterpret_cast<T*>(smem_raw);   // [2][BKV][DK]
  T* Vs = Ks + 2 * BKV * DK;                // [2][DK][BKV]

  // work item: XCD-aware (dispatch is round-robin over 8 XCDs), so one XCD walks
  // consecutive items: all query blocks of a (sequence, head), longest first.
  int item = blockIdx.x;
  if ((n_items & 7) == 0) item = (blockIdx.x & 7) * (n_items >> 3) + (blockIdx.x >> 3);
  const int bh = item / n_qblocks;
  const int qb = n_qblocks - 1 - (item - bh * n_qblocks);
  const int bi = bh / H, head = bh - bi * H;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rho = lane & 31, hf = lane >> 5;
  const int q0 = qb * BQ;
  const int qpos = q0 + wave * 32 + rho;        // this lane's query position
  const size_t seq_row0 = (size_t)bi * N;

  // Q fragments (B operand): lane = query row, 8 consecutive features per k-step
  typename O::frag qf[DK / 16];
#pragma unroll
  for (int ks = 0; ks < DK / 16; ++ks) {
    if (qpos < N) {
      qf[ks] = ld_frag(Qg + (seq_row0 + qpos) * d + head * DK + ks * 16 + 8 * hf);
    } else {
      float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      qf[ks] = O::from_f32(z);
    }
  }

  const int n_kv = (N + BKV - 1) / BKV;
  const int q_last = min(q0 + BQ, N) - 1;
  const int kv_end = causal ? (q_last / BKV + 1) : n_kv;

  const T* Kseq = Kg + seq_row0 * d + head * DK;
  const T* Vhead = Vt + (size_t)bh * DK * ldv;

  typename Chunk<T>::type kreg[KCH], vreg[VCH];
  auto gload = [&](int kv0) {
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      const int c = tid + NTH * j, krow = c / KCPR, kc = c - krow * KCPR;
      kreg[j] = (kv0 + krow < N) ? ld_chunk(Kseq + (size_t)(kv0 + krow) * d + kc * 8)
                                 : zero_chunk<T>();
    }
#pragma unroll
    for (int j = 0; j < VCH; ++j) {
      const int c = tid + NTH * j, vrow = c / VCPR, vc = c - vrow * VCPR;
      const int p0 = kv0 + vc * 8;
      if (p0 + 8 <= N) {
        vreg[j] = ld_chunk(Vhead + (size_t)vrow * ldv + p0);
      } else {
        typename Chunk<T>::type z = zero_chunk<T>();
        T* zt = reinterpret_cast<T*>(&z);
        for (int e = 0; e < 8; ++e)
          if (p0 + e < N) zt[e] = Vhead[(size_t)vrow * ldv + p0 + e];
        vreg[j] = z;
      }
    }
  };
  auto lstore = [&](int buf) {
    T* ks_ = Ks + buf * BKV * DK;
    T* vs_ = Vs + buf * DK * BKV;
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      const int c = tid + NTH * j, krow = c / KCPR, kc = c - krow * KCPR;
      const int lrow = pi_row(krow);
      st_chunk(ks_ + lrow * DK + ((kc ^ (swz(lrow) & (KCPR - 1))) * 8), kreg[j]);
    }
#pragma unroll
    for (int j = 0; j < VCH; ++j) {
      const int c = tid + NTH * j, vrow = c / VCPR, vc = c - vrow * VCPR;
      const int lrow = pi_row(vrow);
      st_chunk(vs_ + lrow * BKV + ((vc ^ (swz(lrow) & (VCPR - 1))) * 8), vreg[j]);
    }
  };

  f32x16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const int wave_q_first = q0 + wave * 32;

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kb = 0; kb < kv_end; ++kb) {
    const int buf = kb & 1;
    const int kv0 = kb * BKV;
    if (kb + 1 < kv_end) gload(kv0 + BKV);
    // a wave whose 32 rows all precede this block has nothing to add
    const bool active = !(causal && kv0 > wave_q_first + 31);
    if (active) {
      const T* ks_ = Ks + buf * BKV * DK;
      const T* vs_ = Vs + buf * DK * BKV;
      f32x16 s[ST];
#pragma unroll
      for (int t = 0; t < ST; ++t) s[t] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < DK / 16; ++kk) {
        const int ch = 2 * kk + hf;
#pragma unroll
        for (int t = 0; t < ST; ++t) {
          const int row = t * 32 + rho;
          O::mma(s[t], ld_frag(ks_ + row * DK + ((ch ^ (swz(row) & (KCPR - 1))) * 8)), qf[kk]);
        }
      }
      // scale into the log2 domain; mask future keys and keys past the end
      const bool need_mask = (kv0 + BKV > N) || (causal && kv0 + BKV - 1 > wave_q_first);
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < ST; ++t) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float v = s[t][i] * scale_log2e;
          if (need_mask) {
            const int kp = kv0 + t * 32 + c_row_pi(i, hf);
            if (kp >= N || (causal && kp > qpos)) v = -INFINITY;
          }
          s[t][i] = v;
          mx = fmaxf(mx, v);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_new;
      float lsum = 0.f;
      typename O::frag pf[BKV / 16];
#pragma unroll
      for (int t = 0; t < ST; ++t) {
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          float p[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float pe = fast_exp2(s[t][8 * g + e] - m_use);
            if constexpr (sizeof(T) == 2) pe = bf16_round(pe);
            p[e] = pe;
            lsum += pe;
          }
          pf[2 * t + g] = O::from_f32(p);
        }
      }
      l_run = l_run * alpha + lsum;
#pragma unroll
      for (int t = 0; t < DT; ++t) oacc[t] *= alpha;
#pragma unroll
      for (int kk = 0; kk < BKV / 16; ++kk) {
        const int ch = 2 * kk + hf;
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          const int row = t * 32 + rho;
          O::mma(oacc[t], ld_frag(vs_ + row * BKV + ((ch ^ (swz(row) & (VCPR - 1))) * 8)), pf[kk]);
        }
      }
    }
    if (kb + 1 < kv_end) lstore(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
  if (qpos < N) {
    T* orow = Og + (seq_row0 + qpos) * d + head * DK;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = oacc[t][8 * g + e] * inv;
        store8_f32(orow + t * 32 + 16 * g + 8 * hf, v);
      }
    }
  }
}

namespace {

template <typename T, int DK, int BQ, int BKV>
int run_attn(const LayerLaunch& L, hipStream_t s, char* err, size_t n) {
  const int nqb = (L.seq_len + BQ - 1) / BQ;
  const int items = L.batch * L.n_heads * nqb;
  const size_t smem = (size_t)4 * BKV * DK * sizeof(T);
  auto k = attention_kernel<T, DK, BQ, BKV>;
  if (set_smem(k, smem, err, n)) return 1;
  const float scale = 1.4426950408889634f / sqrtf((float)DK);
  hipLaunchKernelGGL(k, dim3(items), dim3(BQ * 2), smem, s, (const T*)L.q, (const T*)L.k,
                     (const T*)L.vt, (T*)L.q, L.seq_len, L.n_heads, L.d_model, L.ldv, L.causal,
                     scale, nqb, items);
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
