// HIP kernels of the BPT layer forward for gfx950, and their launchers.
//
//   ln_stats      per-row mean and 1/sqrt(var + eps) of the layer input (LN1)
//   ln_qkv        [Q K V] = LN1(X) [W_Q W_K W_V]  -- LN applied while staging X
//   attention     per (sequence, head, query block): inner loop over key/value
//                 blocks with the running (m, l, o) online softmax
//   ffn_epilogue  per row tile: y = x + O W_O, LN2, then over d_ff chunks
//                 h = GELU(LN2(y) W_1[:, c]), z += h W_2[c, :]; writes Z
//
// Method: "Blockwise Parallel Transformer — BPT" (aicassindra.com), sections
// "The fused blockwise algorithm" and "Pitfalls and misconceptions" (causal
// block skipping); online softmax as in the FlashAttention paragraph of the
// transformer-cost page (raminaeye.github.io).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdio.h>

#include "bpt_device.hpp"
#include "bpt_internal.h"

namespace bpt {

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ===========================================================================
// LN1 statistics: one wave per row, values held in registers (two-pass).
// ===========================================================================
template <typename TX>
__global__ __launch_bounds__(256) void ln_stats_kernel(const TX* __restrict__ X,
                                                       float2* __restrict__ stats, int rows,
                                                       int d, float eps) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + wave;
  if (row >= rows) return;
  const TX* xr = X + (size_t)row * d;
  const int nch = d >> 3;
  float v[8][8];
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int c = lane + 64 * j;
    if (c < nch) {
      load8_f32(xr + 8 * c, v[j]);
#pragma unroll
      for (int e = 0; e < 8; ++e) s += v[j][e];
    }
  }
  s = wave_sum(s);
  const float mean = s / (float)d;
  float q = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int c = lane + 64 * j;
    if (c < nch) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float t = v[j][e] - mean;
        q += t * t;
      }
    }
  }
  q = wave_sum(q);
  if (lane == 0) stats[row] = make_float2(mean, 1.0f / sqrtf(q / (float)d + eps));
}

// ===========================================================================
// LN1 + QKV projection GEMM.
// Output tile C^T[n, r] (n: output feature in [0, 3d), r: token row); A = weight
// rows (pi order), B = LN1(X) rows, both staged through LDS, double-buffered.
// 4 waves in a 2 x 2 grid, each (BN/2) x (BM/2).
// ===========================================================================
template <typename TX, typename T, int BM, int BN, int BK>
__global__ __launch_bounds__(256, 1) void ln_qkv_kernel(
    const TX* __restrict__ X, const float2* __restrict__ stats, const T* __restrict__ ln_g,
    const T* __restrict__ ln_b, const T* __restrict__ wq, const T* __restrict__ wk,
    const T* __restrict__ wv, T* __restrict__ Qo, T* __restrict__ Ko, T* __restrict__ Vt, int R,
    int d, int N, int H, int dk, int ldv, int n_tiles_n) {
  using O = Op<T>;
  constexpr int CPR = BK / 8;                 // 8-element chunks per staged row
  constexpr int ROWS_PER_PASS = 256 / CPR;    // rows covered by one pass of 256 threads
  constexpr int WCH = BN / ROWS_PER_PASS;     // weight chunks per thread
  constexpr int XCH = BM / ROWS_PER_PASS;     // activation chunks per thread
  constexpr int TN = BN / 64, TR = BM / 64;   // 32x32 tiles per wave
  static_assert(256 % CPR == 0 && BN % ROWS_PER_PASS == 0 && BM % ROWS_PER_PASS == 0, "tile");

  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* Ws = reinterpret_cast<T*>(smem_raw);          // [2][BN][BK]
  T* Xs = Ws + 2 * BN * BK;                        // [2][BM][BK]

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rho = lane & 31, hf = lane >> 5;
  const int wn = wave >> 1, wr = wave & 1;
  const int nt = blockIdx.x % n_tiles_n, rt = blockIdx.x / n_tiles_n;
  const int r0 = rt * BM;
  const int ng0 = nt * BN;                 // first output feature in [0, 3d)
  const int which = ng0 / d;               // 0 Q, 1 K, 2 V
  const int nc0 = ng0 - which * d;         // first column inside that matrix
  const T* W = which == 0 ? wq : (which == 1 ? wk : wv);

  const int kc = tid % CPR;                // this thread's chunk column (fixed)
  const int row_base = tid / CPR;

  // per-thread LN statistics of the rows it stages
  float mean_r[XCH], rstd_r[XCH];
#pragma unroll
  for (int j = 0; j < XCH; ++j) {
    const int r = r0 + row_base + ROWS_PER_PASS * j;
    float2 st = r < R ? stats[r] : make_float2(0.f, 0.f);
    mean_r[j] = st.x;
    rstd_r[j] = st.y;
  }

  typename Chunk<T>::type wreg[WCH];
  float xreg[XCH][8];

  auto gload = [&](int k0) {
#pragma unroll
    for (int j = 0; j < WCH; ++j) {
      const int n = nc0 + row_base + ROWS_PER_PASS * j;
      wreg[j] = ld_chunk(W + (size_t)n * d + k0 + kc * 8);
    }
#pragma unroll
    for (int j = 0; j < XCH; ++j) {
      const int r = r0 + row_base + ROWS_PER_PASS * j;
      if (r < R) {
        load8_f32(X + (size_t)r * d + k0 + kc * 8, xreg[j]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) xreg[j][e] = 0.f;
      }
    }
  };
  auto lstore = [&](int buf, int k0) {
    T* ws = Ws + buf * BN * BK;
    T* xs = Xs + buf * BM * BK;
#pragma unroll
    for (int j = 0; j < WCH; ++j) {
      const int row = row_base + ROWS_PER_PASS * j;
      st_chunk(ws + row * BK + ((kc ^ (swz(row) & (CPR - 1))) * 8), wreg[j]);
    }
    float g[8], b[8];
    load8_f32(ln_g + k0 + kc * 8, g);
    load8_f32(ln_b + k0 + kc * 8, b);
#pragma unroll
    for (int j = 0; j < XCH; ++j) {
      const int row = row_base + ROWS_PER_PASS * j;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (xreg[j][e] - mean_r[j]) * rstd_r[j] * g[e] + b[e];
      *reinterpret_cast<typename O::frag*>(xs + row * BK + ((kc ^ (swz(row) & (CPR - 1))) * 8)) =
          O::from_f32(v);
    }
  };

  f32x16 acc[TN][TR];
#pragma unroll
  for (int a = 0; a < TN; ++a)
#pragma unroll
    for (int b = 0; b < TR; ++b) acc[a][b] = f32x16{};

  const int nk = d / BK;
  gload(0);
  lstore(0, 0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
    const T* ws = Ws + buf * BN * BK;
    const T* xs = Xs + buf * BM * BK;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int ch = 2 * ks + hf;
      typename O::frag af[TN], bfr[TR];
#pragma unroll
      for (int a = 0; a < TN; ++a) {
        const int row = wn * (BN / 2) + a * 32 + pi_row(rho);
        af[a] = ld_frag(ws + row * BK + ((ch ^ (swz(row) & (CPR - 1))) * 8));
      }
#pragma unroll
      for (int b = 0; b < TR; ++b) {
        const int row = wr * (BM / 2) + b * 32 + rho;
        bfr[b] = ld_frag(xs + row * BK + ((ch ^ (swz(row) & (CPR - 1))) * 8));
      }
#pragma unroll
      for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int b = 0; b < TR; ++b) O::mma(acc[a][b], af[a], bfr[b]);
    }
    if (kt + 1 < nk) lstore(buf ^ 1, (kt + 1) * BK);
    __syncthreads();
  }

  // epilogue: lane owns token row r and, per 8-register group, 8 consecutive n
#pragma unroll
  for (int b = 0; b < TR; ++b) {
    const int r = r0 + wr * (BM / 2) + b * 32 + rho;
    if (r >= R) continue;
    const int bi = r / N, pos = r - bi * N;
#pragma unroll
    for (int a = 0; a < TN; ++a) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int n = nc0 + wn * (BN / 2) + a * 32 + 16 * g + 8 * hf;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = acc[a][b][8 * g + e];
        if (which < 2) {
          store8_f32((which == 0 ? Qo : Ko) + (size_t)r * d + n, v);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int col = n + e, head = col / dk, j = col - head * dk;
            Vt[((size_t)(bi * H + head) * dk + j) * ldv + pos] = (T)v[e];
          }
        }
      }
    }
  }
}

// ===========================================================================
// Attention: one workgroup per (sequence, head, query block of BQ rows), one
// wave per 32 query rows. S^T = K Q^T and O^T += V^T P^T on the matrix cores,
// so each lane owns one query row: row max / row sum are in-lane plus one
// exchange between the two lane halves. K and V^T tiles are staged in LDS,
// double-buffered. Causal: key blocks past the query block are never visited.
// ===========================================================================
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

// ===========================================================================
// Fused epilogue of one row tile of BM tokens:
//   Y^T = W_O O^T + X^T           (fp32, registers; wave w owns features
//                                   [w D/4, (w+1) D/4) of all BM rows)
//   LN2(Y) -> LDS (compute type)
//   for each chunk of HC hidden units:
//     U^T = W_1[chunk] LN2(Y)^T   (each wave HC/4 hidden units)
//     H   = GELU(U) -> LDS        (the [BM, HC] tile; never leaves the CU)
//     Z^T += W_2[:, chunk] H^T
//   Z = Y + H W_2 written once.
// ===========================================================================
template <typename TX, typename T, typename TO, int D, int BM, int HC>
__global__ __launch_bounds__(256, 1) void ffn_epilogue_kernel(
    const TX* X, const T* __restrict__ Oin, const T* __restrict__ wo,
    const T* __restrict__ ln_g, const T* __restrict__ ln_b, const T* __restrict__ w1,
    const T* __restrict__ w2, TO* Z, int R, int dff, float eps) {
  using O = Op<T>;
  constexpr int NCW = D / 4;       // features per wave
  constexpr int NT = NCW / 32;     // 32-feature tiles per wave
  constexpr int RT = BM / 32;      // 32-row tiles
  constexpr int FT = HC / 4 / 32;  // hidden tiles per wave per chunk
  constexpr int YCPR = D / 8, HCPR = HC / 8;
  static_assert(NT >= 1 && RT >= 1 && FT >= 1, "tile");

  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* Ys = reinterpret_cast<T*>(smem_raw);     // [BM][D]: O tile, then LN2(Y)
  T* Hs = Ys + BM * D;                        // [BM][HC]: hidden chunk
  float* red = reinterpret_cast<float*>(Hs);  // [2][4][BM] row partial sums (before the FFN)

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rho = lane & 31, hf = lane >> 5;
  const int r0 = blockIdx.x * BM;
  const int n0w = wave * NCW;

  // ---- stage the attention-output tile O[r0 : r0 + BM, :] in LDS
  for (int c = tid; c < BM * YCPR; c += 256) {
    const int row = c / YCPR, cc = c - row * YCPR;
    const int r = r0 + row;
    auto v = r < R ? ld_chunk(Oin + (size_t)r * D + cc * 8) : zero_chunk<T>();
    st_chunk(Ys + row * D + ((cc ^ swz(row)) * 8), v);
  }
  __syncthreads();

  // ---- Y^T = W_O O^T
  f32x16 acc[NT][RT];
#pragma unroll
  for (int a = 0; a < NT; ++a)
#pragma unroll
    for (int b = 0; b < RT; ++b) acc[a][b] = f32x16{};
  for (int ks = 0; ks < D / 16; ++ks) {
    const int ch = 2 * ks + hf;
    typename O::frag af[NT], bfr[RT];
#pragma unroll
    for (int a = 0; a < NT; ++a)
      af[a] = ld_frag(wo + (size_t)(n0w + a * 32 + pi_row(rho)) * D + ks * 16 + 8 * hf);
#pragma unroll
    for (int b = 0; b < RT; ++b) {
      const int row = b * 32 + rho;
      bfr[b] = ld_frag(Ys + row * D + ((ch ^ swz(row)) * 8));
    }
#pragma unroll
    for (int a = 0; a < NT; ++a)
#pragma unroll
      for (int b = 0; b < RT; ++b) O::mma(acc[a][b], af[a], bfr[b]);
  }
  // ---- + X (residual), and this wave's partial row sums
  float psum[RT];
#pragma unroll
  for (int b = 0; b < RT; ++b) {
    const int r = r0 + b * 32 + rho;
    float s = 0.f;
#pragma unroll
    for (int a = 0; a < NT; ++a) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        float xv[8];
        if (r < R) {
          load8_f32(X + (size_t)r * D + n0w + a * 32 + 16 * g + 8 * hf, xv);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) xv[e] = 0.f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          acc[a][b][8 * g + e] += xv[e];
          s += acc[a][b][8 * g + e];
        }
      }
    }
    psum[b] = s + __shfl_xor(s, 32, 64);
  }
  __syncthreads();  // every wave is done reading the O tile (Ys) and may reuse Hs
  if (hf == 0) {
#pragma unroll
    for (int b = 0; b < RT; ++b) red[wave * BM + b * 32 + rho] = psum[b];
  }
  __syncthreads();
  float mean[RT], rstd[RT];
#pragma unroll
  for (int b = 0; b < RT; ++b) {
    const int row = b * 32 + rho;
    mean[b] = (red[row] + red[BM + row] + red[2 * BM + row] + red[3 * BM + row]) / (float)D;
    float q = 0.f;
#pragma unroll
    for (int a = 0; a < NT; ++a)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float t = acc[a][b][i] - mean[b];
        q += t * t;
      }
    psum[b] = q + __shfl_xor(q, 32, 64);
  }
  if (hf == 0) {
#pragma unroll
    for (int b = 0; b < RT; ++b) red[4 * BM + wave * BM + b * 32 + rho] = psum[b];
  }
  __syncthreads();
#pragma unroll
  for (int b = 0; b < RT; ++b) {
    const int row = b * 32 + rho;
    const float q = red[4 * BM + row] + red[5 * BM + row] + red[6 * BM + row] + red[7 * BM + row];
    rstd[b] = 1.0f / sqrtf(q / (float)D + eps);
  }
  // ---- LN2(Y) -> Ys (compute type), 8 consecutive features per store
#pragma unroll
  for (int a = 0; a < NT; ++a) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int n = n0w + a * 32 + 16 * g + 8 * hf;
      float gv[8], bv[8];
      load8_f32(ln_g + n, gv);
      load8_f32(ln_b + n, bv);
#pragma unroll
      for (int b = 0; b < RT; ++b) {
        const int row = b * 32 + rho;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (acc[a][b][8 * g + e] - mean[b]) * rstd[b] * gv[e] + bv[e];
        *reinterpret_cast<typename O::frag*>(Ys + row * D + (((n >> 3) ^ swz(row)) * 8)) =
            O::from_f32(v);
      }
    }
  }
  __syncthreads();

  // ---- FFN over hidden chunks
  const int n_chunks = dff / HC;
  for (int c = 0; c < n_chunks; ++c) {
    const int f0 = c * HC + wave * (HC / 4);
    f32x16 u[FT][RT];
#pragma unroll
    for (int a = 0; a < FT; ++a)
#pragma unroll
      for (int b = 0; b < RT; ++b) u[a][b] = f32x16{};
    for (int ks = 0; ks < D / 16; ++ks) {
      const int ch = 2 * ks + hf;
      typename O::frag af[FT], bfr[RT];
#pragma unroll
      for (int a = 0; a < FT; ++a)
        af[a] = ld_frag(w1 + (size_t)(f0 + a * 32 + pi_row(rho)) * D + ks * 16 + 8 * hf);
#pragma unroll
      for (int b = 0; b < RT; ++b) {
        const int row = b * 32 + rho;
        bfr[b] = ld_frag(Ys + row * D + ((ch ^ swz(row)) * 8));
      }
#pragma unroll
      for (int a = 0; a < FT; ++a)
#pragma unroll
        for (int b = 0; b < RT; ++b) O::mma(u[a][b], af[a], bfr[b]);
    }
    // GELU -> Hs
#pragma unroll
    for (int a = 0; a < FT; ++a) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int fl = wave * (HC / 4) + a * 32 + 16 * g + 8 * hf;   // hidden unit within chunk
#pragma unroll
        for (int b = 0; b < RT; ++b) {
          const int row = b * 32 + rho;
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = gelu_tanh(u[a][b][8 * g + e]);
          *reinterpret_cast<typename O::frag*>(Hs + row * HC + (((fl >> 3) ^ (swz(row) & (HCPR - 1))) * 8)) =
              O::from_f32(v);
        }
      }
    }
    __syncthreads();
    // Z^T += W_2[:, chunk] H^T
    for (int ks = 0; ks < HC / 16; ++ks) {
      const int ch = 2 * ks + hf;
      typename O::frag af[NT], bfr[RT];
#pragma unroll
      for (int a = 0; a < NT; ++a)
        af[a] = ld_frag(w2 + (size_t)(n0w + a * 32 + pi_row(rho)) * dff + c * HC + ks * 16 + 8 * hf);
#pragma unroll
      for (int b = 0; b < RT; ++b) {
        const int row = b * 32 + rho;
        bfr[b] = ld_frag(Hs + row * HC + ((ch ^ (swz(row) & (HCPR - 1))) * 8));
      }
#pragma unroll
      for (int a = 0; a < NT; ++a)
#pragma unroll
        for (int b = 0; b < RT; ++b) O::mma(acc[a][b], af[a], bfr[b]);
    }
    __syncthreads();
  }

  // ---- Z = Y + H W_2
#pragma unroll
  for (int b = 0; b < RT; ++b) {
    const int r = r0 + b * 32 + rho;
    if (r >= R) continue;
#pragma unroll
    for (int a = 0; a < NT; ++a) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = acc[a][b][8 * g + e];
        store8_f32(Z + (size_t)r * D + n0w + a * 32 + 16 * g + 8 * hf, v);
      }
    }
  }
}

// ===========================================================================
// Launchers
// ===========================================================================
namespace {

void set_err(char* err, size_t n, const char* fmt, const char* a = "", int b = 0) {
  if (err && n) snprintf(err, n, fmt, a, b);
}

template <typename K>
int set_smem(K kernel, size_t bytes, char* err, size_t errlen) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e != hipSuccess) {
    set_err(err, errlen, "hipFuncSetAttribute: %s", hipGetErrorString(e));
    return 1;
  }
  return 0;
}

int check_launch(const char* what, char* err, size_t errlen) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    if (err && errlen) snprintf(err, errlen, "%s launch: %s", what, hipGetErrorString(e));
    return 1;
  }
  return 0;
}

// ---- LN1 statistics
template <typename TX>
int run_stats(const LayerLaunch& L, hipStream_t s, char* err, size_t n) {
  const int rows = L.batch * L.seq_len;
  hipLaunchKernelGGL(ln_stats_kernel<TX>, dim3((rows + 3) / 4), dim3(256), 0, s,
                     (const TX*)L.x, (float2*)L.stats, rows, L.d_model, L.ln_eps);
  return check_launch("ln_stats", err, n);
}

// ---- LN1 + QKV
template <typename TX, typename T, int BM, int BN, int BK>
int run_qkv(const LayerLaunch& L, hipStream_t s, char* err, size_t n) {
  const int rows = L.batch * L.seq_len;
  const int ntn = 3 * L.d_model / BN;
  const int ntr = (rows + BM - 1) / BM;
  const size_t smem = (size_t)2 * (BM + BN) * BK * sizeof(T);
  auto k = ln_qkv_kernel<TX, T, BM, BN, BK>;
  if (set_smem(k, smem, err, n)) return 1;
  hipLaunchKernelGGL(k, dim3(ntn * ntr), dim3(256), smem, s, (const TX*)L.x,
                     (const float2*)L.stats, (const T*)L.w.ln1_g, (const T*)L.w.ln1_b,
                     (const T*)L.w.w_q, (const T*)L.w.w_k, (const T*)L.w.w_v, (T*)L.q, (T*)L.k,
                     (T*)L.vt, rows, L.d_model, L.seq_len, L.n_heads, L.d_head, L.ldv, ntn);
  return check_launch("ln_qkv", err, n);
}

// ---- attention
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

// ---- FFN epilogue
template <typename TX, typename T, typename TO, int D, int BM, int HC>
int run_ffn(const LayerLaunch& L, hipStream_t s, char* err, size_t n) {
  const int rows = L.batch * L.seq_len;
  const size_t smem = (size_t)BM * (D + HC) * sizeof(T);
  auto k = ffn_epilogue_kernel<TX, T, TO, D, BM, HC>;
  if (set_smem(k, smem, err, n)) return 1;
  hipLaunchKernelGGL(k, dim3((rows + BM - 1) / BM), dim3(256), smem, s, (const TX*)L.x,
                     (const T*)L.q, (const T*)L.w.w_o, (const T*)L.w.ln2_g, (const T*)L.w.ln2_b,
                     (const T*)L.w.w_1, (const T*)L.w.w_2, (TO*)L.z, rows, L.d_ff, L.ln_eps);
  return check_launch("ffn_epilogue", err, n);
}

template <typename TX, typename T, typename TO>
int dispatch_ffn(const LayerLaunch& L, hipStream_t s, char* err, size_t n) {
  const int d = L.d_model;
  if constexpr (sizeof(T) == 4) {
    if (d == 128) return run_ffn<TX, T, TO, 128, 64, 256>(L, s, err, n);
    if (d == 256) return run_ffn<TX, T, TO, 256, 32, 256>(L, s, err, n);
  } else {
    if (d == 256) return run_ffn<TX, T, TO, 256, 64, 256>(L, s, err, n);
    if (d == 512) return run_ffn<TX, T, TO, 512, 64, 256>(L, s, err, n);
    if (d == 768) return run_ffn<TX, T, TO, 768, 64, 256>(L, s, err, n);
    if (d == 1024) return run_ffn<TX, T, TO, 1024, 64, 256>(L, s, err, n);
    if (d == 2048) return run_ffn<TX, T, TO, 2048, 32, 256>(L, s, err, n);
  }
  set_err(err, n, "no epilogue kernel for d_model %s%d", "", d);
  return 1;
}

int mark(const LayerLaunch& L, int i, hipStream_t s, char* err, size_t n) {
  if (!L.events) return 0;
  hipError_t e = hipEventRecord(reinterpret_cast<hipEvent_t>(L.events[i]), s);
  if (e != hipSuccess) {
    set_err(err, n, "hipEventRecord: %s", hipGetErrorString(e));
    return 1;
  }
  return 0;
}

template <typename TX, typename T>
int run_layer_typed(const LayerLaunch& L, hipStream_t s, char* err, size_t n) {
  if (mark(L, 0, s, err, n) || run_stats<TX>(L, s, err, n) || mark(L, 1, s, err, n)) return 1;
  if constexpr (sizeof(T) == 2) {
    if (run_qkv<TX, T, 256, 256, 64>(L, s, err, n)) return 1;
  } else {
    if (run_qkv<TX, T, 128, 128, 32>(L, s, err, n)) return 1;
  }
  if (mark(L, 2, s, err, n) || dispatch_attn<T>(L, s, err, n) || mark(L, 3, s, err, n)) return 1;
  const int r = L.z_f32 ? dispatch_ffn<TX, T, float>(L, s, err, n)
                        : dispatch_ffn<TX, T, bf16>(L, s, err, n);
  return r || mark(L, 4, s, err, n);
}

}  // namespace

int launch_layer(const LayerLaunch& L, void* stream, char* err, size_t errlen) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (L.compute_f32) return run_layer_typed<float, float>(L, s, err, errlen);
  if (L.x_f32) return run_layer_typed<float, bf16>(L, s, err, errlen);
  return run_layer_typed<bf16, bf16>(L, s, err, errlen);
}

}  // namespace bpt
