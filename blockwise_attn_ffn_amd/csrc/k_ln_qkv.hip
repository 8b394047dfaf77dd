// LN1 statistics and the LN1 + QKV projection GEMM (gfx950).
//
// "Blockwise Parallel Transformer — BPT" (aicassindra.com), section "The fused
// blockwise algorithm": q_i = LN(x_i) W_Q and k_j, v_j = LN(X[j]) W_K, LN(X[j]) W_V.
// Here K and V are projected once for all rows instead of once per inner-loop
// visit; the values are the same.
#include "bpt_device.hpp"
#include "bpt_launch.hpp"

namespace bpt {

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ---------------------------------------------------------------------------
// LN1 statistics: one wave per row, the row held in registers (two passes:
// mean, then the biased variance of the centred values).
// ---------------------------------------------------------------------------
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

// ---------------------------------------------------------------------------
// LN1 + QKV projection GEMM.
// Output tile C^T[n, r] (n: output feature in [0, 3d), r: token row); A = weight
// rows (pi order), B = LN1(X) rows; both staged through LDS, double-buffered,
// with the next k-tile's global loads in flight during the current one.
// 4 waves in a 2 x 2 grid, each (BN/2) x (BM/2).
// ---------------------------------------------------------------------------
template <typename TX, typename T, int BM, int BN, int BK>
__global__ __launch_bounds__(256, 1) void ln_qkv_kernel(
    const TX* __restrict__ X, const float2* __restrict__ stats, const T* __restrict__ ln_g,
    const T* __restrict__ ln_b, const T* __restrict__ wq, const T* __restrict__ wk,
    const T* __restrict__ wv, T* __restrict__ Qo, T* __restrict__ Ko, T* __restrict__ Vt, int R,
    int d, int N, int H, int dk, int ldv, int n_tiles_n) {
  using O = Op<T>;
  using F = typename O::frag;
  constexpr int CPR = BK / 8;                 // 8-element chunks per staged row
  constexpr int ROWS_PER_PASS = 256 / CPR;    // rows covered by one pass of 256 threads
  constexpr int WCH = BN / ROWS_PER_PASS;     // weight chunks per thread
  constexpr int XCH = BM / ROWS_PER_PASS;     // activation chunks per thread
  constexpr int TN = BN / 64, TR = BM / 64;   // 32x32 tiles per wave
  constexpr int KS = BK / 16;
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

  // Rows past the end are clamped to the last row: their results are never stored.
  float mean_r[XCH], rstd_r[XCH];
  const TX* xrow[XCH];
#pragma unroll
  for (int j = 0; j < XCH; ++j) {
    const int r = min(r0 + row_base + ROWS_PER_PASS * j, R - 1);
    const float2 st = stats[r];
    mean_r[j] = st.x;
    rstd_r[j] = st.y;
    xrow[j] = X + (size_t)r * d + kc * 8;
  }
  const T* wrow = W + (size_t)(nc0 + row_base) * d + kc * 8;

  typename Chunk<T>::type wreg[WCH];
  float xreg[XCH][8];

  auto gload = [&](int k0) {
#pragma unroll
    for (int j = 0; j < WCH; ++j) wreg[j] = ld_chunk(wrow + (size_t)ROWS_PER_PASS * j * d + k0);
#pragma unroll
    for (int j = 0; j < XCH; ++j) load8_f32(xrow[j] + k0, xreg[j]);
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
      *reinterpret_cast<F*>(xs + row * BK + ((kc ^ (swz(row) & (CPR - 1))) * 8)) = O::from_f32(v);
    }
  };
  auto lfrags = [&](const T* ws, const T* xs, int ks, F (&af)[TN], F (&bf)[TR]) {
    const int ch = 2 * ks + hf;
#pragma unroll
    for (int a = 0; a < TN; ++a) {
      const int row = wn * (BN / 2) + a * 32 + pi_row(rho);
      af[a] = ld_frag(ws + row * BK + ((ch ^ (swz(row) & (CPR - 1))) * 8));
    }
#pragma unroll
    for (int b = 0; b < TR; ++b) {
      const int row = wr * (BM / 2) + b * 32 + rho;
      bf[b] = ld_frag(xs + row * BK + ((ch ^ (swz(row) & (CPR - 1))) * 8));
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
    F af[2][TN], bf[2][TR];
    lfrags(ws, xs, 0, af[0], bf[0]);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) lfrags(ws, xs, ks + 1, af[(ks + 1) & 1], bf[(ks + 1) & 1]);
#pragma unroll
      for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int b = 0; b < TR; ++b) O::mma(acc[a][b], af[ks & 1][a], bf[ks & 1][b]);
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
          // V^T[seq, head, j, pos]: 8 consecutive j of one head, stride ldv
          const int head = n / dk, j0 = n - head * dk;
          T* vp = Vt + ((size_t)(bi * H + head) * dk + j0) * ldv + pos;
#pragma unroll
          for (int e = 0; e < 8; ++e) vp[(size_t)e * ldv] = (T)v[e];
        }
      }
    }
  }
}

namespace {

template <typename TX>
int run_stats(const LayerLaunch& L, hipStream_t s, char* err, size_t n) {
  const int rows = L.batch * L.seq_len;
  hipLaunchKernelGGL(ln_stats_kernel<TX>, dim3((rows + 3) / 4), dim3(256), 0, s,
                     (const TX*)L.x, (float2*)L.stats, rows, L.d_model, L.ln_eps);
  return check_launch("ln_stats", err, n);
}

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

}  // namespace

// phase 0: LN1 statistics; phase 1: the projection GEMM.
int launch_ln_qkv(const LayerLaunch& L, hipStream_t s, char* err, size_t n, int phase) {
  if (phase == 0) {
    if (L.x_f32) return run_stats<float>(L, s, err, n);
    return L.compute_f32 ? run_stats<float>(L, s, err, n) : run_stats<bf16>(L, s, err, n);
  }
  if (L.compute_f32) return run_qkv<float, float, 128, 128, 32>(L, s, err, n);
  if (L.x_f32) return run_qkv<float, bf16, 256, 256, 64>(L, s, err, n);
  return run_qkv<bf16, bf16, 256, 256, 64>(L, s, err, n);
}

}  // namespace bpt
