// LN1 and the QKV projection GEMM (gfx950).
//
// "Blockwise Parallel Transformer — BPT" (aicassindra.com), section "The fused
// blockwise algorithm": q_i = LN(x_i) W_Q and k_j, v_j = LN(X[j]) W_K, LN(X[j]) W_V.
// K and V are projected once for all rows instead of once per inner-loop visit;
// the values are the same.
//
// Rows are handled in "packed row" space: sequence b occupies packed rows
// [b Np, b Np + N) with Np = N rounded up to 128; the padding rows are zero.
// ln_pack: per row, LN1 statistics (mean, biased variance, two passes over the
//   row held in registers) and LN1(x) = (x - mean) / sqrt(var + eps) * g + b,
//   written once in the compute type as matrix-core B fragments (packed order,
//   bpt_device.hpp) -- the GEMM's activation operand.
// qkv_gemm: C^T[3d, rows] = [W_Q W_K W_V] LN1(X)^T with both operands packed;
//   256 x 256 tiles, operands copied global -> LDS by the LDS-DMA path into two
//   static LDS stages (no register staging), the next k-tile in flight while the
//   current one is multiplied. Q, K and V are written as the attention kernel's
//   packed operands (k_attention.hip).
#include <type_traits>

#include "bpt_device.hpp"
#include "bpt_launch.hpp"

namespace bpt {

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ---------------------------------------------------------------------------
// LN1 into packed B fragments, rows fed through pi: slot s of a fragment holds
// packed row pi(s % 32) of its 32-row tile (so that the QKV product can emit the
// V^T operand directly, see below). One workgroup per 32-row tile: the four
// waves first compute the row statistics (8 rows each, rows read coalesced),
// then write the tile's fragments one 1 KB fragment per wave instruction.
// Rows of a sequence's padding and rows in [R, Rp) are zero.
// ---------------------------------------------------------------------------
template <typename TX, typename T, int CPL>
__global__ __launch_bounds__(256) void ln_pack_kernel(const TX* __restrict__ X,
                                                      const T* __restrict__ ln_g,
                                                      const T* __restrict__ ln_b,
                                                      T* __restrict__ XP, int B, int N, int Np,
                                                      int d, float eps) {
  // CPL: 8-element chunks per lane per row (d <= 512 CPL)
  __shared__ float2 stats[32];           // (mean, rstd); rstd = 0 marks a zero row
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tile = blockIdx.x;
  const int nch = d >> 3, KS = d >> 4;
#pragma unroll 2
  for (int i = 0; i < 8; ++i) {
    const int r = wave + 4 * i, row = tile * 32 + r;
    const int bi = row / Np, pos = row - bi * Np;
    float mean = 0.f, rstd = 0.f;
    if (bi < B && pos < N) {
      const TX* xr = X + ((size_t)bi * N + pos) * d;
      float v[CPL][8];
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const int c = lane + 64 * j;
        if (c < nch) {
          load8_f32(xr + 8 * c, v[j]);
#pragma unroll
          for (int e = 0; e < 8; ++e) sum += v[j][e];
        }
      }
      mean = wave_sum(sum) / (float)d;
      float q = 0.f;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const int c = lane + 64 * j;
        if (c < nch) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float t = v[j][e] - mean;
            q += t * t;
          }
        }
      }
      rstd = 1.0f / sqrtf(wave_sum(q) / (float)d + eps);
    }
    if (lane == 0) stats[r] = make_float2(mean, rstd);
  }
  __syncthreads();
  // fragment ks: lane (hf, s) holds row pi(s) and k = 16 ks + 8 hf + [0, 8)
  const int rr = pi_row(lane & 31), hf = lane >> 5;
  const int row = tile * 32 + rr;
  const int bi = row / Np, pos = row - bi * Np;
  const float2 st = stats[rr];
  const bool live = st.y != 0.f;
  const TX* xr = X + ((size_t)bi * N + min(pos, N - 1)) * d;
  T* out = XP + (size_t)tile * KS * kFragElems;
  for (int ks = wave; ks < KS; ks += 4) {
    const int k0 = 16 * ks + 8 * hf;
    float v[8];
    if (live) {
      float x[8], g[8], b[8];
      load8_f32(xr + k0, x);
      load8_f32(ln_g + k0, g);
      load8_f32(ln_b + k0, b);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (x[e] - st.x) * st.y * g[e] + b[e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
    st_packed(out + (size_t)ks * kFragElems, lane, v);
  }
}

// LDS-staged variant (d <= 2048): eight waves read the tile's 32 rows once
// (4 rows each, coalesced), normalise them in registers and write the packed
// fragments into LDS; the tile then leaves LDS for global memory as contiguous
// 16-byte chunks. X is read exactly once.
template <typename TX, typename T, int CPL>
__global__ __launch_bounds__(512) void ln_pack_lds_kernel(const TX* __restrict__ X,
                                                          const T* __restrict__ ln_g,
                                                          const T* __restrict__ ln_b,
                                                          T* __restrict__ XP, int B, int N, int Np,
                                                          int d, float eps) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* tile_lds = reinterpret_cast<T*>(smem_raw);          // [d/16] packed fragments
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tile = blockIdx.x;
  const int nch = d >> 3;
#pragma unroll 2
  for (int i = 0; i < 4; ++i) {
    const int r = wave + 8 * i, row = tile * 32 + r;
    const int bi = row / Np, pos = row - bi * Np;
    const bool live = bi < B && pos < N;
    float v[CPL][8];
    if (live) {
      const TX* xr = X + ((size_t)bi * N + pos) * d;
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const int c = lane + 64 * j;
        if (c < nch) {
          load8_f32(xr + 8 * c, v[j]);
#pragma unroll
          for (int e = 0; e < 8; ++e) sum += v[j][e];
        }
      }
      const float mean = wave_sum(sum) / (float)d;
      float q = 0.f;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const int c = lane + 64 * j;
        if (c < nch) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float t = v[j][e] - mean;
            q += t * t;
          }
        }
      }
      const float rstd = 1.0f / sqrtf(wave_sum(q) / (float)d + eps);
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const int c = lane + 64 * j;
        if (c < nch) {
          float g[8], b[8];
          load8_f32(ln_g + 8 * c, g);
          load8_f32(ln_b + 8 * c, b);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[j][e] = (v[j][e] - mean) * rstd * g[e] + b[e];
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < CPL; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) v[j][e] = 0.f;
    }
    // chunk c (k = 8c .. 8c+7) of row r: fragment c/2, slot 32 (c&1) + pi(r)
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + 64 * j;
      if (c < nch) st_packed(tile_lds + (size_t)(c >> 1) * kFragElems, 32 * (c & 1) + pi_row(r), v[j]);
    }
  }
  __syncthreads();
  const int n16 = (32 * d * (int)sizeof(T)) >> 4;         // 16-byte chunks in the tile
  const uint4* src = reinterpret_cast<const uint4*>(tile_lds);
  uint4* dst = reinterpret_cast<uint4*>(XP + (size_t)tile * 32 * d);
  for (int q = threadIdx.x; q < n16; q += 512) dst[q] = src[q];
}

// ---------------------------------------------------------------------------
// QKV GEMM on packed operands. Tile BN output features x BM token rows; 4 waves
// in a 2 x 2 grid, each (BN/2) x (BM/2) as 32x32 tiles. A k-tile is 4 k-steps.
// LDS stage = [A: BN/32 tiles][4 k-steps][fragment] then [B: BM/32 tiles][...].
// ---------------------------------------------------------------------------
template <typename T, int BN, int BM>
__global__ __launch_bounds__(256, 1) void qkv_gemm_kernel(
    const T* __restrict__ WP, const T* __restrict__ XP, T* __restrict__ Qo, T* __restrict__ Ko,
    T* __restrict__ Vt, int rows_used, int d, int Np, int H, int dk, int n_tiles_n) {
  // Qo: B fragments over [packed rows, d]; Ko: per (sequence, head) A fragments
  // over [Np keys (pi order), d_k]; Vt: per (sequence, head) A fragments over
  // [d_k (pi order), Np keys].
  using O = Op<T>;
  using F = typename O::frag;
  constexpr int PCS = frag_pieces<T>();
  constexpr int FB = 1024 * PCS;                    // bytes per fragment
  constexpr int TA = BN / 32, TB = BM / 32;         // 32-row tiles per operand
  constexpr int STAGE_A = TA * 4 * FB, STAGE = (TA + TB) * 4 * FB;
  constexpr int NCOPY = (TA + TB) * 4 * PCS;        // 1 KB copies per k-tile
  constexpr int CPW = NCOPY / 4;                    // per wave
  constexpr int TN = TA / 2, TR = TB / 2;           // 32x32 tiles per wave
  static_assert(NCOPY % 4 == 0, "copies per wave");
  __shared__ __align__(16) unsigned char lds0[STAGE];
  __shared__ __align__(16) unsigned char lds1[STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rho = lane & 31, hf = lane >> 5;
  const int wn = wave >> 1, wr = wave & 1;
  // Tile order: dispatch is round-robin over the 8 XCDs, so consecutive workgroup
  // ids are renumbered to give each XCD a contiguous range of tiles, and inside
  // that range tiles run in groups of G row tiles per column tile: the ~32
  // workgroups an XCD runs at once share G row tiles and few column tiles of the
  // operands in its L2.
  int id = blockIdx.x;
  const int n_tiles = gridDim.x;
  if ((n_tiles & 7) == 0) id = (id & 7) * (n_tiles >> 3) + (id >> 3);
  constexpr int G = 8;
  const int n_tiles_r = n_tiles / n_tiles_n;
  const int grp = id / (G * n_tiles_n), in_grp = id - grp * G * n_tiles_n;
  const int g_rows = min(G, n_tiles_r - grp * G);
  const int rt = grp * G + in_grp % g_rows, nt = in_grp / g_rows;
  const int KS = d / 16, nk = d / 64;

  // Copy k-tile kt into an LDS stage: wave w issues copies [w CPW, (w+1) CPW).
  auto issue = [&](int kt, unsigned char* buf) {
#pragma unroll
    for (int q = 0; q < CPW; ++q) {
      const int idx = wave * CPW + q;
      const int piece = idx % PCS, f = idx / PCS;
      const bool is_a = f < TA * 4;
      const int ff = is_a ? f : f - TA * 4;
      const int tile = ff >> 2, ksl = ff & 3;
      const size_t frag = (size_t)((is_a ? nt * TA : rt * TB) + tile) * KS + kt * 4 + ksl;
      const T* src = (is_a ? WP : XP) + frag * kFragElems + piece * (kFragElems / PCS);
      dma16(src + lane * (8 / PCS), buf + f * FB + piece * 1024);
    }
  };

  f32x16 acc[TN][TR];
#pragma unroll
  for (int a = 0; a < TN; ++a)
#pragma unroll
    for (int b = 0; b < TR; ++b) acc[a][b] = f32x16{};

  // swap = false: acc[a][b] = C^T tile (rows: features, cols: tokens);
  // swap = true:  acc[a][b] = C tile   (rows: tokens, cols: features).
  // The fragments of k-step ksl+1 are read from LDS while the products of k-step
  // ksl run (two register sets), so LDS latency is hidden inside a k-tile.
  auto compute = [&](const unsigned char* buf, auto swap) {
    F af[2][TN], bfr[2][TR];
    auto load = [&](int ksl, F (&a_)[TN], F (&b_)[TR]) {
#pragma unroll
      for (int a = 0; a < TN; ++a)
        a_[a] = ld_packed(reinterpret_cast<const T*>(buf + ((wn * TN + a) * 4 + ksl) * FB), lane);
#pragma unroll
      for (int b = 0; b < TR; ++b)
        b_[b] = ld_packed(
            reinterpret_cast<const T*>(buf + STAGE_A + ((wr * TR + b) * 4 + ksl) * FB), lane);
    };
    load(0, af[0], bfr[0]);
#pragma unroll
    for (int ksl = 0; ksl < 4; ++ksl) {
      const int cs = ksl & 1;
      if (ksl < 3) load(ksl + 1, af[cs ^ 1], bfr[cs ^ 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int b = 0; b < TR; ++b) {
          if constexpr (decltype(swap)::value) O::mma(acc[a][b], bfr[cs][b], af[cs][a]);
          else O::mma(acc[a][b], af[cs][a], bfr[cs][b]);
        }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // nk is even (d is a multiple of 128): the two stages alternate with constant names.
  auto main_loop = [&](auto swap) {
    issue(0, lds0);
    for (int kt = 0; kt < nk; kt += 2) {
      wait_vmem();
      __syncthreads();           // stage 0 landed for every wave; stage 1 is free
      issue(kt + 1, lds1);
      compute(lds0, swap);
      wait_vmem();
      __syncthreads();           // stage 1 landed; stage 0 is free
      if (kt + 2 < nk) issue(kt + 2, lds0);
      compute(lds1, swap);
    }
  };

  const int ng0 = nt * BN;                 // first output feature in [0, 3d)
  const int which = ng0 / d;               // 0 Q, 1 K, 2 V
  const int nc0 = ng0 - which * d;         // first column inside that matrix
  const int KSD = dk / 16;
  if (which != 2) {
    main_loop(std::false_type{});
    // lane (hf, rho) holds packed row pi(rho) of its tile and, per register group
    // g, the 8 consecutive features 16 g + 8 hf + [0, 8) of its feature tile
#pragma unroll
    for (int b = 0; b < TR; ++b) {
      const int p = rt * BM + wr * (BM / 2) + b * 32 + pi_row(rho);
      if (p >= rows_used) continue;
      const int bi = p / Np, pos = p - bi * Np;
#pragma unroll
      for (int a = 0; a < TN; ++a) {
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const int n = nc0 + wn * (BN / 2) + a * 32 + 16 * g + 8 * hf;
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = acc[a][b][8 * g + e];
          if (which == 0) {
            st_packed(Qo + ((size_t)(p >> 5) * KS + (n >> 4)) * kFragElems, 32 * hf + (p & 31), v);
          } else {
            const int head = n / dk, j0 = n - head * dk;
            const size_t frag = (((size_t)bi * H + head) * (Np / 32) + (pos >> 5)) * KSD + (j0 >> 4);
            st_packed(Ko + frag * kFragElems, 32 * hf + pi_row(pos & 31), v);   // = lane
          }
        }
      }
    }
  } else {
    main_loop(std::true_type{});
    // lane (hf, rho) holds feature pi(rho) of its feature tile and, per register
    // group g, the 8 consecutive tokens 16 g + 8 hf + [0, 8) of its token tile:
    // one V^T fragment slot (feature pi(rho), 8 consecutive keys) per group.
#pragma unroll
    for (int b = 0; b < TR; ++b) {
      const int p0 = rt * BM + wr * (BM / 2) + b * 32;   // first token of the tile
      if (p0 >= rows_used) continue;
      const int bi = p0 / Np, pos0 = p0 - bi * Np;        // a tile lies inside one sequence
#pragma unroll
      for (int a = 0; a < TN; ++a) {
        const int n0 = nc0 + wn * (BN / 2) + a * 32;      // first feature of the tile
        const int head = n0 / dk, dt = (n0 - head * dk) >> 5;
        T* vbase = Vt + ((((size_t)bi * H + head) * (dk / 32) + dt) * (Np / 16) + (pos0 >> 4)) * kFragElems;
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = acc[a][b][8 * g + e];
          st_packed(vbase + (size_t)g * kFragElems, lane, v);
        }
      }
    }
  }
}

namespace {

template <typename TX, typename T>
int run_ln_pack(const LayerLaunch& L, hipStream_t s, char* err, size_t n) {
  const int d = L.d_model;
  if (d <= 2048) {
    auto k = d <= 512 ? ln_pack_lds_kernel<TX, T, 1>
                      : (d <= 1024 ? ln_pack_lds_kernel<TX, T, 2> : ln_pack_lds_kernel<TX, T, 4>);
    const size_t smem = (size_t)32 * d * sizeof(T);
    if (set_smem(k, smem, err, n)) return 1;
    hipLaunchKernelGGL(k, dim3(L.rows_pad / 32), dim3(512), smem, s, (const TX*)L.x,
                       (const T*)L.w.ln1_g, (const T*)L.w.ln1_b, (T*)L.xpack, L.batch, L.seq_len,
                       L.seq_pad, d, L.ln_eps);
    return check_launch("ln_pack", err, n);
  }
  auto k = ln_pack_kernel<TX, T, 8>;
  hipLaunchKernelGGL(k, dim3(L.rows_pad / 32), dim3(256), 0, s, (const TX*)L.x, (const T*)L.w.ln1_g,
                     (const T*)L.w.ln1_b, (T*)L.xpack, L.batch, L.seq_len, L.seq_pad, d, L.ln_eps);
  return check_launch("ln_pack", err, n);
}

template <typename T, int BN, int BM>
int run_qkv(const LayerLaunch& L, hipStream_t s, char* err, size_t n) {
  const int ntn = 3 * L.d_model / BN;
  const int ntr = L.rows_pad / BM;
  hipLaunchKernelGGL((qkv_gemm_kernel<T, BN, BM>), dim3(ntn * ntr), dim3(256), 0, s,
                     (const T*)L.wpack, (const T*)L.xpack, (T*)L.q, (T*)L.k, (T*)L.vt,
                     L.batch * L.seq_pad, L.d_model, L.seq_pad, L.n_heads, L.d_head, ntn);
  return check_launch("qkv_gemm", err, n);
}

}  // namespace

// phase 0: LN1 into the packed operand; phase 1: the projection GEMM.
int launch_ln_qkv(const LayerLaunch& L, hipStream_t s, char* err, size_t n, int phase) {
  if (phase == 0) {
    if (L.compute_f32) return run_ln_pack<float, float>(L, s, err, n);
    return L.x_f32 ? run_ln_pack<float, bf16>(L, s, err, n) : run_ln_pack<bf16, bf16>(L, s, err, n);
  }
  if (L.compute_f32) return run_qkv<float, 128, 128>(L, s, err, n);
  return run_qkv<bf16, 256, 256>(L, s, err, n);
}

}  // namespace bpt
