// Matrix products of the layer on packed operands (gfx950): the QKV projection
// and the row-block FFN (Y = X + O W_O, LN2, then per block of rows W_1 -> GELU
// -> W_2), which serves the shapes neither fused epilogue takes: bf16 pairs up
// to d_model 1024, and wide layers whose d_ff is not a multiple of the
// cooperative epilogue's chunk.
//
// "Blockwise Parallel Transformer — BPT" (aicassindra.com), section "The fused
// blockwise algorithm": the queries of a block come from its LN1 rows through
// W_Q, its keys and values from LN1 of the key rows through W_K and W_V (here
// projected once for all rows instead of once per inner-loop visit; the values
// are the same), and a block is finished by W_O with the residual, LN, the FFN
// and the second residual.
//
// One kernel, C^T = W A^T on packed fragments, 256 x 256 tiles (bf16: 8 waves,
// two per SIMD, each 128 features x 64 rows), operands copied global -> LDS by
// the LDS-DMA path into two static stages (the next k-tile in flight while the
// current one is multiplied), the next k-step's fragments read from LDS during
// the current k-step's products, XCD-contiguous grouped tile order. The epilogue mode decides the output:
//   kModeQKV:    Q (packed B fragments), K and V^T (the attention kernel's operands);
//   kModeResidY: Y = X + O W_O, fp32 row-major over packed rows;
//   kModeGeluH:  GELU(LN2(Y) W_1) for a block of rows, as packed B fragments;
//   kModeOutZ:   Z = Y + H W_2, real rows, Z's element type.
// In the staged epilogue the hidden state exists only for one block of rows at a
// time (a bounded workspace block), never for all rows.
#include <type_traits>

#include "bpt_device.hpp"
#include "bpt_launch.hpp"

namespace bpt {

enum GemmMode { kModeQKV = 0, kModeResidY = 1, kModeGeluH = 2, kModeOutZ = 3 };

template <typename T>
struct GemmArgs {
  const T* w;          // weight fragments [features, K], plain order
  const T* a;          // activation B fragments [rows, K] (starting at row0)
  const T* a_lo;       // optional lo half of a bf16 pair operand: C += W a_lo^T too
  int K, n_tiles_n, row0, a_pi;   // a_pi: rows of a are pi-ordered inside a tile
  int N, Np, rows_used;           // sequence geometry of packed rows
  // kModeQKV
  T *q, *k, *vt;
  T *q_lo, *k_lo, *vt_lo;         // optional lo halves of the outputs
  int d, H, dk;
  int G, dkv, kvp;                // key/value heads, their width, that width padded to BN
  // other modes
  int n_out;                      // features of the output row
  const void* x;                  // residual X (real rows), kModeResidY
  int x_f32;
  float* y;                       // Y, kModeResidY output / kModeOutZ input
  T* h;                           // hidden block, kModeGeluH output
  T* h_lo;                        // optional lo half
  void* z;                        // Z (real rows), kModeOutZ
  int z_f32;
};

// ---------------------------------------------------------------------------
// C^T[features, rows] = W[features, K] . A[rows, K]^T on packed operands: W in
// plain fragment order (k_pack.hip), A as packed B fragments. Tile BN features x
// BM rows; NW waves in a 2 x (NW/2) grid, each (BN/2) x (BM/(NW/2)) as 32x32
// tiles (NW = 8: two waves per SIMD, so one wave's copy issue and barrier waits
// are covered by the other's products). A k-tile is 4 k-steps. LDS stage = [W: BN/32 tiles][4 k-steps][fragment] then
// [A: BM/32 tiles][...]. The epilogue (MODE) decides what the tile becomes.
// ---------------------------------------------------------------------------
template <typename T, int BN, int BM, int MODE, int NW>
__global__ __launch_bounds__(64 * NW, 1) void gemm_kernel(GemmArgs<T> g) {
  using O = Op<T>;
  using F = typename O::frag;
  constexpr int PCS = frag_pieces<T>();
  constexpr int FB = 1024 * PCS;                    // bytes per fragment
  constexpr int TA = BN / 32, TB = BM / 32;         // 32-row tiles per operand
  constexpr int STAGE_A = TA * 4 * FB, STAGE = (TA + TB) * 4 * FB;
  constexpr int NCOPY = (TA + TB) * 4 * PCS;        // 1 KB copies per k-tile
  constexpr int WR = NW / 2;                        // waves along the rows
  constexpr int CPW = NCOPY / NW;                   // per wave
  constexpr int TN = TA / 2, TR = TB / WR;          // 32x32 tiles per wave
  static_assert(NCOPY % NW == 0 && TR >= 1 && TB % WR == 0, "copies and tiles per wave");
  __shared__ __align__(16) unsigned char lds0[STAGE];
  __shared__ __align__(16) unsigned char lds1[STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rho = lane & 31, hf = lane >> 5;
  const int wn = wave / WR, wr = wave % WR;
  // Tile order: dispatch is round-robin over the 8 XCDs, so consecutive workgroup
  // ids are renumbered to give each XCD a contiguous range of tiles, and inside
  // that range tiles run in groups of G row tiles per column tile: the ~32
  // workgroups an XCD runs at once share G row tiles and few column tiles of the
  // operands in its L2.
  int id = blockIdx.x;
  const int n_tiles = gridDim.x;
  if ((n_tiles & 7) == 0) id = (id & 7) * (n_tiles >> 3) + (id >> 3);
  constexpr int G = 8;
  const int n_tiles_n = g.n_tiles_n;
  const int n_tiles_r = n_tiles / n_tiles_n;
  const int grp = id / (G * n_tiles_n), in_grp = id - grp * G * n_tiles_n;
  const int g_rows = min(G, n_tiles_r - grp * G);
  const int rt = grp * G + in_grp % g_rows, nt = in_grp / g_rows;
  // with a lo operand the k-loop runs twice over K: W a^T, then W a_lo^T
  const int KS = g.K / 16, nk1 = g.K / 64, nk = g.a_lo ? 2 * nk1 : nk1;
  const T* __restrict__ WP = g.w;
  const T* __restrict__ XP = g.a;

  // Copy k-tile kt into an LDS stage: wave w issues copies [w CPW, (w+1) CPW). With
  // square tiles the first half of the waves copy W and the others A, so a wave has one
  // source base; copy q's byte offset in k-tile 0 is loop-invariant (k-tile kw adds
  // kw * 4 fragments), and so is its LDS destination.
  static_assert(TA == TB, "square tiles: the first NW/2 waves copy W, the others A");
  const bool w_copier = wave < NW / 2;
  uint32_t c_off[CPW];
#pragma unroll
  for (int q = 0; q < CPW; ++q) {
    const int idx = wave * CPW + q;
    const int piece = idx % PCS, f = idx / PCS;
    const int ff = w_copier ? f : f - TA * 4;
    const int tile = ff >> 2, ksl = ff & 3;
    const uint32_t frag = (uint32_t)((w_copier ? nt * TA : rt * TB) + tile) * KS + ksl;
    c_off[q] = (frag * kFragElems + piece * (kFragElems / PCS)) * (uint32_t)sizeof(T);
  }
  const uint32_t lane_off = (uint32_t)lane * 16u;
  auto issue_one = [&](int kt, unsigned char* buf, int q) __attribute__((always_inline)) {
    const int idx = wave * CPW + q;
    const int piece = idx % PCS, f = idx / PCS;
    const bool lo = kt >= nk1;
    const uint32_t kw = (uint32_t)(lo ? kt - nk1 : kt);
    const char* base = reinterpret_cast<const char*>(w_copier ? WP : (lo ? g.a_lo : XP));
    dma16(base + (c_off[q] + kw * (4u * kFragElems * (uint32_t)sizeof(T)) + lane_off),
          buf + f * FB + piece * 1024);
  };
  auto issue = [&](int kt, unsigned char* buf) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < CPW; ++q) issue_one(kt, buf, q);
  };

  f32x16 acc[TN][TR];
#pragma unroll
  for (int a = 0; a < TN; ++a)
#pragma unroll
    for (int b = 0; b < TR; ++b) acc[a][b] = f32x16{};

  // swap = false: acc[a][b] = C^T tile (rows: features, cols: tokens);
  // swap = true:  acc[a][b] = C tile   (rows: tokens, cols: features).
  // The fragments of k-step ksl+1 are read from LDS while the products of k-step
  // ksl run (two register sets), so LDS latency is hidden inside a k-tile. The
  // copies of the next k-tile (has_next) into nbuf are issued among the first
  // k-step's products, so their address arithmetic runs in the products' shadow.
  auto compute = [&](const unsigned char* buf, auto swap, auto has_next, int kt_next,
                     unsigned char* nbuf) __attribute__((always_inline)) {
    constexpr bool kNext = decltype(has_next)::value;
    F af[2][TN], bfr[2][TR];
    auto load = [&](int ksl, F (&a_)[TN], F (&b_)[TR]) __attribute__((always_inline)) {
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
          constexpr int kPer = CPW / (TN * TR) > 0 ? CPW / (TN * TR) : 1;
          const int q0 = (a * TR + b) * kPer;
          if (kNext && ksl == 0 && q0 < CPW) {
#pragma unroll
            for (int q = 0; q < kPer; ++q)
              if (q0 + q < CPW) issue_one(kt_next, nbuf, q0 + q);
          }
        }
      if (kNext && ksl == 0) {
#pragma unroll
        for (int q = TN * TR * (CPW / (TN * TR) > 0 ? CPW / (TN * TR) : 1); q < CPW; ++q)
          issue_one(kt_next, nbuf, q);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // nk is even (K is a multiple of 128): the two stages alternate with constant names;
  // the last k-tile issues no copies.
  auto main_loop = [&](auto swap) __attribute__((always_inline)) {
    issue(0, lds0);
    for (int kt = 0; kt < nk - 2; kt += 2) {
      wait_vmem();
      __syncthreads();           // stage 0 landed for every wave; stage 1 is free
      compute(lds0, swap, std::true_type{}, kt + 1, lds1);
      wait_vmem();
      __syncthreads();           // stage 1 landed; stage 0 is free
      compute(lds1, swap, std::true_type{}, kt + 2, lds0);
    }
    wait_vmem();
    __syncthreads();
    compute(lds0, swap, std::true_type{}, nk - 1, lds1);
    wait_vmem();
    __syncthreads();
    compute(lds1, swap, std::false_type{}, -1, lds0);
  };

  // Non-swapped tiles: lane (hf, rho) holds packed row row0 + ... + r(rho) of its
  // tile, r = pi(rho) when the A operand's rows are pi-ordered, and per register
  // group gg the 8 consecutive features 16 gg + 8 hf + [0, 8) of its feature tile.
  auto row_of = [&](int b) {
    return g.row0 + rt * BM + wr * (BM / WR) + b * 32 + (g.a_pi ? pi_row(rho) : rho);
  };
  auto frag_vals = [&](const f32x16& t, int gg, float* v) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = t[8 * gg + e];
  };
  // store v at (hi + off), and its residual v - bf16(v) at (lo + off) when lo is set
  auto st_pair = [&](T* hi, T* lo, size_t off, int slot, float* v) {
    st_packed(hi + off, slot, v);
    if (lo) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] -= bf16_round(v[e]);
      st_packed(lo + off, slot, v);
    }
  };
  const int Np = g.Np;
  if constexpr (MODE == kModeQKV) {
    const int d = g.d, dk = g.dk, G = g.G, dkv = g.dkv, kvp = g.kvp, rows_used = g.rows_used;
    const int ng0 = nt * BN;                 // first output feature in [0, d + 2 kvp)
    // 0 Q, 1 K, 2 V: d and kvp are multiples of BN, so a tile lies inside one part;
    // K and V features at or past dkv (the padding) are not stored
    const int which = ng0 < d ? 0 : (ng0 < d + kvp ? 1 : 2);
    const int nc0 = ng0 - (which == 0 ? 0 : (which == 1 ? d : d + kvp));   // column inside it
    const int KSD = dk / 16, KSQ = d / 16;
    if (which != 2) {
      main_loop(std::false_type{});
#pragma unroll
      for (int b = 0; b < TR; ++b) {
        const int p = row_of(b);
        if (p >= rows_used) continue;
        const int bi = p / Np, pos = p - bi * Np;
#pragma unroll
        for (int a = 0; a < TN; ++a) {
#pragma unroll
          for (int gg = 0; gg < 2; ++gg) {
            const int n = nc0 + wn * (BN / 2) + a * 32 + 16 * gg + 8 * hf;
            float v[8];
            frag_vals(acc[a][b], gg, v);
            if (which == 0) {
              st_pair(g.q, g.q_lo, ((size_t)(p >> 5) * KSQ + (n >> 4)) * kFragElems, 32 * hf + (p & 31), v);
            } else if (n < dkv) {
              const int head = n / dk, j0 = n - head * dk;
              const size_t frag = (((size_t)bi * G + head) * (Np / 32) + (pos >> 5)) * KSD + (j0 >> 4);
              st_pair(g.k, g.k_lo, frag * kFragElems, 32 * hf + pi_row(pos & 31), v);   // = lane
            }
          }
        }
      }
    } else {
      main_loop(std::true_type{});
      // lane (hf, rho) holds feature pi(rho) of its feature tile and, per register
      // group gg, the 8 consecutive tokens 16 gg + 8 hf + [0, 8) of its token tile
      // (rows pi-ordered): one V^T fragment slot (feature pi(rho), 8 consecutive
      // keys) per group.
#pragma unroll
      for (int b = 0; b < TR; ++b) {
        const int p0 = g.row0 + rt * BM + wr * (BM / WR) + b * 32;  // first token of the tile
        if (p0 >= rows_used) continue;
        const int bi = p0 / Np, pos0 = p0 - bi * Np;        // a tile lies inside one sequence
#pragma unroll
        for (int a = 0; a < TN; ++a) {
          const int n0 = nc0 + wn * (BN / 2) + a * 32;      // first feature of the tile
          if (n0 >= dkv) continue;                           // padding features
          const int head = n0 / dk, dt = (n0 - head * dk) >> 5;
          const size_t vbase = ((((size_t)bi * G + head) * (dk / 32) + dt) * (Np / 16) + (pos0 >> 4)) * kFragElems;
#pragma unroll
          for (int gg = 0; gg < 2; ++gg) {
            float v[8];
            frag_vals(acc[a][b], gg, v);
            st_pair(g.vt, g.vt_lo, vbase + (size_t)gg * kFragElems, lane, v);
          }
        }
      }
    }
  } else {
    main_loop(std::false_type{});
    const int n_out = g.n_out;               // row length of the output
#pragma unroll
    for (int b = 0; b < TR; ++b) {
      const int p = row_of(b);
      if (p >= g.rows_used) continue;
      const int bi = p / Np, pos = p - bi * Np;
#pragma unroll
      for (int a = 0; a < TN; ++a) {
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
          const int n = nt * BN + wn * (BN / 2) + a * 32 + 16 * gg + 8 * hf;
          float v[8];
          frag_vals(acc[a][b], gg, v);
          if constexpr (MODE == kModeResidY) {
            // Y = X + C over packed rows (padding rows: C alone), fp32 row-major
            if (pos < g.N) {
              float x[8];
              const size_t xr = ((size_t)bi * g.N + pos) * n_out + n;
              if (g.x_f32) load8_f32(static_cast<const float*>(g.x) + xr, x);
              else load8_f32(static_cast<const bf16*>(g.x) + xr, x);
#pragma unroll
              for (int e = 0; e < 8; ++e) v[e] += x[e];
            }
            store8_f32(g.y + (size_t)p * n_out + n, v);
          } else if constexpr (MODE == kModeGeluH) {
            // H = GELU(C) as packed B fragments over [block rows, d_ff]; the row
            // order of the operand carries over (slot = lane)
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = gelu_tanh(v[e]);
            const int pl = p - g.row0;
            st_pair(g.h, g.h_lo, ((size_t)(pl >> 5) * (n_out / 16) + (n >> 4)) * kFragElems, lane, v);
          } else {
            // Z = Y + C, real rows only
            if (pos >= g.N) continue;
            float y[8];
            load8_f32(g.y + (size_t)p * n_out + n, y);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] += y[e];
            const size_t zr = ((size_t)bi * g.N + pos) * n_out + n;
            if (g.z_f32) store8_f32(static_cast<float*>(g.z) + zr, v);
            else store8_f32(static_cast<bf16*>(g.z) + zr, v);
          }
        }
      }
    }
  }
}

namespace {

template <typename T, int BN, int BM, int MODE, int NW = (sizeof(T) == 2 ? 8 : 4)>
int run_gemm(const GemmArgs<T>& g, int n_feat, int rows, hipStream_t s, const char* what, char* err,
             size_t n) {
  // copy offsets are 32-bit byte offsets from each operand's base
  const unsigned long long kMaxBytes = 1ull << 32;
  if ((unsigned long long)n_feat * g.K * sizeof(T) >= kMaxBytes ||
      (unsigned long long)rows * g.K * sizeof(T) >= kMaxBytes) {
    set_err(err, n, "%s: an operand of 4 GiB or more is not supported", what);
    return 1;
  }
  GemmArgs<T> a = g;
  a.n_tiles_n = n_feat / BN;
  const int ntr = rows / BM;
  hipLaunchKernelGGL((gemm_kernel<T, BN, BM, MODE, NW>), dim3(a.n_tiles_n * ntr), dim3(64 * NW), 0, s, a);
  return check_launch(what, err, n);
}

template <typename T, int BN, int BM>
int run_qkv(const LayerLaunch& L, hipStream_t s, char* err, size_t n) {
  GemmArgs<T> g{};
  g.w = static_cast<const T*>(L.wpack);
  g.a = static_cast<const T*>(L.xpack);
  g.K = L.d_model;
  g.row0 = 0;
  g.a_pi = 1;
  g.N = L.seq_len;
  g.Np = L.seq_pad;
  g.rows_used = L.batch * L.seq_pad;
  g.q = static_cast<T*>(L.q);
  g.k = static_cast<T*>(L.k);
  g.vt = static_cast<T*>(L.vt);
  if (L.split) {
    g.a_lo = static_cast<const T*>(L.xpack_lo);
    g.q_lo = static_cast<T*>(L.q_lo);
    g.k_lo = static_cast<T*>(L.k_lo);
    g.vt_lo = static_cast<T*>(L.vt_lo);
  }
  g.d = L.d_model;
  g.H = L.n_heads;
  g.dk = L.d_head;
  g.G = L.n_kv_heads;
  g.dkv = L.d_kv;
  g.kvp = L.kv_pad;
  if (L.d_model % BN != 0 || L.kv_pad % BN != 0) {
    set_err(err, n, "qkv product: widths not multiples of the %s%d-feature tile", "", BN);
    return 1;
  }
  return run_gemm<T, BN, BM, kModeQKV>(g, L.d_model + 2 * L.kv_pad, L.rows_pad, s, "qkv_gemm", err,
                                       n);
}

}  // namespace

int launch_qkv(const LayerLaunch& L, hipStream_t s, char* err, size_t n) {
  if (L.compute_f32) return run_qkv<float, 128, 128>(L, s, err, n);
  return run_qkv<bf16, 256, 256>(L, s, err, n);
}

// Staged epilogue (bf16): Y = X + O W_O (fp32, over the dead K/V^T buffers), LN2(Y)
// packed (over the dead LN1 operand), then per block of h_rows rows
// H = GELU(LN2(Y) W_1) into the hidden block and Z = Y + H W_2. With split (bf16
// pairs) every activation operand is a (hi, lo) pair and each product runs over
// both halves.
int launch_ffn_staged(const LayerLaunch& L, hipStream_t s, char* err, size_t n) {
  using T = bf16;
  if (L.compute_f32) {
    set_err(err, n, "the staged epilogue has no fp32 instance%s", "");
    return 1;
  }
  const int d = L.d_model, f = L.d_ff;
  const size_t dd = (size_t)d * d, qkv = qkv_pack_elems(d, L.kv_pad);
  const T* wp = static_cast<const T*>(L.wpack);
  GemmArgs<T> g{};
  g.N = L.seq_len;
  g.Np = L.seq_pad;
  g.rows_used = L.batch * L.seq_pad;
  g.x = L.x;
  g.x_f32 = L.x_f32;
  g.y = static_cast<float*>(L.ybuf);
  g.z = L.z;
  g.z_f32 = L.z_f32;
  // Y = X + O W_O; O's rows are in natural order inside a tile
  g.w = wp + qkv;
  g.a = static_cast<const T*>(L.q);
  g.a_lo = L.split ? static_cast<const T*>(L.q_lo) : nullptr;
  g.K = d;
  g.row0 = 0;
  g.a_pi = 0;
  g.n_out = d;
  if (run_gemm<T, 256, 256, kModeResidY>(g, d, L.rows_pad, s, "wo_gemm", err, n)) return 1;
  if (launch_ln_rows(L, L.ybuf, L.rows_pad, s, err, n)) return 1;   // LN2(Y) -> xpack (pi rows)
  for (int r0 = 0; r0 < L.rows_pad; r0 += L.h_rows) {
    const int rows = L.rows_pad - r0 < L.h_rows ? L.rows_pad - r0 : L.h_rows;
    GemmArgs<T> u = g;
    u.w = wp + qkv + dd;
    u.a = static_cast<const T*>(L.xpack) + (size_t)(r0 / 32) * (d / 16) * kFragElems;
    u.a_lo = L.split ? static_cast<const T*>(L.xpack_lo) + (size_t)(r0 / 32) * (d / 16) * kFragElems
                     : nullptr;
    u.K = d;
    u.row0 = r0;
    u.a_pi = 1;
    u.n_out = f;
    u.h = static_cast<T*>(L.hbuf);
    u.h_lo = L.split ? static_cast<T*>(L.hbuf_lo) : nullptr;
    if (run_gemm<T, 256, 256, kModeGeluH>(u, f, rows, s, "w1_gemm", err, n)) return 1;
    GemmArgs<T> o = g;
    o.w = wp + qkv + dd + (size_t)f * d;
    o.a = static_cast<const T*>(L.hbuf);
    o.a_lo = L.split ? static_cast<const T*>(L.hbuf_lo) : nullptr;
    o.K = f;
    o.row0 = r0;
    o.a_pi = 1;
    o.n_out = d;
    if (run_gemm<T, 256, 256, kModeOutZ>(o, d, rows, s, "w2_gemm", err, n)) return 1;
  }
  return 0;
}

}  // namespace bpt
