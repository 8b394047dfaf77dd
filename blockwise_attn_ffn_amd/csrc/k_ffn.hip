// Fused per-row-tile epilogue of the BPT layer (gfx950): output projection,
// residual, LN2, FFN W_1 -> GELU -> W_2 and the second residual.
//
// "Blockwise Parallel Transformer — BPT" (aicassindra.com): section "The fused
// blockwise algorithm" (each query block's attention output is finished by the
// output projection and residual, then LN and the FFN, whose hidden state is
// discarded once the block's output rows exist) and "The structural fact that
// makes fusion legal" (LN, the FFN and the residuals act on each row alone, so
// a row tile can be finished as soon as its attention output exists).
//
// One workgroup = BM token rows, 4 waves. Wave w owns output features
// [w D/4, (w+1) D/4) of all BM rows; their fp32 accumulators stay in registers
// from Y through Z. The [BM, d_ff] hidden state is produced and consumed in
// chunks of HC units, each chunk living only in registers and LDS.
//
// The weights arrive as one linear stream per wave (ffn_stream.hpp): W_O, then
// per chunk W_1[chunk] and W_2[chunk], each stage one 32-row tile x 4 k-steps in
// matrix-core fragment order. Stages stream from L2 into a ring of P register
// stages that runs continuously across the phases, so the loads of later stages
// are in flight while the matrix cores work. The residual X initialises the
// accumulators, so Y = X + O W_O leaves the matrix cores complete.
#include <type_traits>

#include "bpt_device.hpp"
#include "bpt_launch.hpp"
#include "ffn_stream.hpp"

namespace bpt {

// LDS holds the [BM, K] activation operands (the O tile, then LN2(Y), with
// K = d; the hidden chunk with K = HC) as packed matrix-core B fragments,
// row tiles interleaved: fragment (row tile b, k-step ks) at (ks * RT + b) * 512
// elements, 64 lanes x 8 consecutive elements in lane order. A k-block's
// fragments are adjacent, so a lane reaches them from one base register with
// immediate offsets, and 64 lanes read 1 KB contiguously.

template <typename TX, typename T, typename TO, int D, int BM, int P>
__global__ __launch_bounds__(256, 1) void ffn_epilogue_kernel(
    const TX* X, const T* __restrict__ Opk, const T* __restrict__ ws,
    const T* __restrict__ ln_g, const T* __restrict__ ln_b, TO* Z, int N, int Np, int dff,
    float eps) {
  // X, Z: [batch * N, d] real rows. Opk: the attention output as packed B fragments
  // over [packed rows, d] (sequence b at packed rows [b Np, b Np + N)). A tile of
  // BM packed rows lies inside one sequence (BM divides Np).
  using O = Op<T>;
  using F = typename O::frag;
  constexpr int HC = kFfnChunk;
  constexpr FfnStream FS{D, 0};
  constexpr int NCW = D / kFfnWaves;     // features per wave
  constexpr int NT = FS.nt();            // 32-feature tiles per wave
  constexpr int RT = BM / 32;            // 32-row tiles
  constexpr int FT = FS.ft();            // hidden tiles per wave per chunk
  constexpr int KBO = D / 64;            // k-blocks when k runs over d (W_O, W_1)
  constexpr int KB2 = HC / 64;           // k-blocks when k runs over a chunk (W_2)
  constexpr int PCS = frag_pieces<T>();
  constexpr int SA = 4;                  // fragments per stage
  constexpr int STAGE = SA * kFragElems; // elements per stage
  // Y/Z tiles that move to ordinary registers while the W_1 accumulators need the
  // accumulator registers (at most 256 of them per lane).
  constexpr int ACC_REGS = (NT + FT) * RT * 16;
  constexpr int PARK = ACC_REGS > 256 ? (ACC_REGS - 256 + 15) / 16 : 0;
  static_assert(NT >= 1 && RT >= 1 && FT >= 1 && D % 128 == 0, "tile");
  static_assert(P == 2 || P == 4, "ring depth");
  static_assert(PARK <= NT * RT, "parked tiles");
  static_assert(8 * BM * 4 + 2 * D * (int)sizeof(T) <= BM * HC * (int)sizeof(T),
                "LN2 scratch must fit in the hidden-chunk buffer");
  static_assert((RT * (D / 16) * PCS) % kFfnWaves == 0, "O-tile copies per wave");

  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* ys = reinterpret_cast<T*>(smem_raw);       // [D/16][RT] fragments: O tile, then LN2(Y)
  T* hs = ys + BM * D;                          // [HC/16][RT] fragments: hidden chunk
  float* red = reinterpret_cast<float*>(hs);    // [2][4][BM] row partial sums
  T* gb = reinterpret_cast<T*>(red + 8 * BM);   // [2][D] LN2 gain and bias (as given)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
  const int rho = lane & 31, hf = lane >> 5;
  const int r0 = blockIdx.x * BM;              // first packed row of the tile
  const int seq = r0 / Np, pos0 = r0 - seq * Np;
  const int n0w = wave * NCW;
  const int n_chunks = dff / HC;
  const int n_stages = FS.n_wo() + n_chunks * FS.per_chunk();
  const T* stream = ws + (size_t)wave * n_stages * STAGE;

  // Stage t of this wave's stream; stages past the end reload the last one, so
  // every call issues the same SA loads and the memory-counter waits stay exact.
  auto load_stage = [&](int t, F (&dst)[SA]) {
    const T* base = stream + (size_t)min(t, n_stages - 1) * STAGE;
#pragma unroll
    for (int j = 0; j < SA; ++j) dst[j] = ld_packed(base + j * kFragElems, lane);
  };

  // ---- the attention-output tile: RT row tiles x D/16 fragments, contiguous per
  //      row tile in Opk, copied global -> LDS (row tiles interleaved) by the
  //      LDS-DMA path, one 1 KB piece per instruction
  {
    constexpr int NC = RT * (D / 16) * PCS, CPW = NC / kFfnWaves;
    const T* src0 = Opk + (size_t)(r0 >> 5) * (D / 16) * kFragElems;
#pragma unroll 4
    for (int q = 0; q < CPW; ++q) {
      const int idx = wave * CPW + q;       // = (row tile * D/16 + k-step) * PCS + piece
      const int b = idx / ((D / 16) * PCS), rest = idx - b * ((D / 16) * PCS);
      const int ks = rest / PCS, piece = rest - ks * PCS;
      dma16(src0 + (size_t)idx * (kFragElems / PCS) + lane * (8 / PCS),
            reinterpret_cast<unsigned char*>(ys) + ((ks * RT + b) * PCS + piece) * 1024);
    }
  }
  F ring[P][SA];
  int t_next = 0;
#pragma unroll
  for (int p = 0; p < P; ++p) load_stage(t_next++, ring[p]);
  for (int c = tid; c < D / 8; c += 256) {
    st_chunk(gb + 8 * c, ld_chunk(ln_g + 8 * c));
    st_chunk(gb + D + 8 * c, ld_chunk(ln_b + 8 * c));
  }
  // Accumulators start at the residual X (fp32). Register group g of feature tile
  // a holds features a*32 + 16g + 8hf + [0, 8) of row rho. Padding rows read a
  // clamped real row; their results are never stored.
  f32x16 acc[NT][RT];
#pragma unroll
  for (int b = 0; b < RT; ++b) {
    const int pos = min(pos0 + b * 32 + rho, N - 1);
    const TX* xr = X + ((size_t)seq * N + pos) * D + n0w + 8 * hf;
#pragma unroll
    for (int a = 0; a < NT; ++a)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        float xv[8];
        load8_f32(xr + a * 32 + 16 * g, xv);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[a][b][8 * g + e] = xv[e];
      }
  }
  wait_vmem();
  __syncthreads();

  // One GEMM phase: accs[tile][r] += A(ring stages) * B(LDS k-blocks of src).
  // Stages run k-block major. The B fragments of a k-block are held in registers
  // for its TT stages; during the last stage each k-step's fragments are reloaded
  // in place with the next k-block's as soon as they have been used.
  auto gemm_phase = [&](const T* src, int n_kb, auto& accs, auto tiles_c) {
    constexpr int TT = decltype(tiles_c)::value;
    // k-blocks unrolled together so that the ring slot of every stage is static
    constexpr int U = (TT % P == 0) ? 1 : ((2 * TT) % P == 0 ? 2 : 4);
    F bq[4][RT];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int b = 0; b < RT; ++b) bq[j][b] = ld_packed(src + (size_t)(j * RT + b) * kFragElems, lane);
    for (int kb0 = 0; kb0 < n_kb; kb0 += U) {
#pragma unroll
      for (int ku = 0; ku < U; ++ku) {
        const T* next = src + (size_t)min(kb0 + ku + 1, n_kb - 1) * (4 * RT * kFragElems);
#pragma unroll
        for (int a = 0; a < TT; ++a) {
          const int p = (ku * TT + a) % P;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int b = 0; b < RT; ++b) O::mma(accs[a][b], ring[p][j], bq[j][b]);
            if (a == TT - 1) {
#pragma unroll
              for (int b = 0; b < RT; ++b)
                bq[j][b] = ld_packed(next + (size_t)(j * RT + b) * kFragElems, lane);
              // issue each reload right after its last use: ~6 products of latency
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          load_stage(t_next++, ring[p]);
          // keep the ring as written: the loads of stage t+P are issued here, P
          // stages before their use, and not sunk towards it by the scheduler
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };

  // Keep the last PARK Y/Z tiles in ordinary registers across a W_1 phase.
  auto park = [&]() {
#pragma unroll
    for (int q = NT * RT - PARK; q < NT * RT; ++q) asm volatile("" : "+v"(acc[q / RT][q % RT]));
  };
  // Pin every Y/Z tile to the accumulator registers (the LN2 arithmetic reads
  // them through transient copies instead of moving them out).
  auto pin = [&]() {
#pragma unroll
    for (int q = 0; q < NT * RT; ++q) asm volatile("" : "+a"(acc[q / RT][q % RT]));
  };

  // ---- Y^T = X^T + W_O O^T
  gemm_phase(ys, KBO, acc, std::integral_constant<int, NT>{});
  pin();

  // ---- LN2 statistics (biased variance, two passes)
  float psum[RT];
#pragma unroll
  for (int b = 0; b < RT; ++b) {
    float s = 0.f;
#pragma unroll
    for (int a = 0; a < NT; ++a)
#pragma unroll
      for (int i = 0; i < 16; ++i) s += acc[a][b][i];
    psum[b] = s + __shfl_xor(s, 32, 64);
  }
  pin();   // each LN2 pass reads the tiles afresh (no long-lived copies)
  if (hf == 0) {
#pragma unroll
    for (int b = 0; b < RT; ++b) red[wave * BM + b * 32 + rho] = psum[b];
  }
  __syncthreads();  // partial sums visible; every wave is done reading the O tile
  float mean[RT], rstd[RT];
#pragma unroll
  for (int b = 0; b < RT; ++b) {
    const int row = b * 32 + rho;
    mean[b] = (red[row] + red[BM + row] + red[2 * BM + row] + red[3 * BM + row]) * (1.0f / D);
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
  pin();
  if (hf == 0) {
#pragma unroll
    for (int b = 0; b < RT; ++b) red[4 * BM + wave * BM + b * 32 + rho] = psum[b];
  }
  __syncthreads();
#pragma unroll
  for (int b = 0; b < RT; ++b) {
    const int row = b * 32 + rho;
    const float q = red[4 * BM + row] + red[5 * BM + row] + red[6 * BM + row] + red[7 * BM + row];
    rstd[b] = 1.0f / sqrtf(q * (1.0f / D) + eps);
  }
  // ---- LN2(Y) -> ys (compute type), 8 consecutive features per store
#pragma unroll
  for (int a = 0; a < NT; ++a) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int n = n0w + a * 32 + 16 * g + 8 * hf;
      float gv[8], bv[8];
      load8_f32(gb + n, gv);
      load8_f32(gb + D + n, bv);
#pragma unroll
      for (int b = 0; b < RT; ++b) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (acc[a][b][8 * g + e] - mean[b]) * rstd[b] * gv[e] + bv[e];
        st_packed(ys + (size_t)((n >> 4) * RT + b) * kFragElems, lane, v);
      }
    }
  }
  pin();
  __syncthreads();

  // ---- FFN over hidden chunks
  for (int c = 0; c < n_chunks; ++c) {
    park();
    // U^T = W_1[chunk] LN2(Y)^T : this wave's HC/4 hidden units of all BM rows
    f32x16 u[FT][RT];
#pragma unroll
    for (int a = 0; a < FT; ++a)
#pragma unroll
      for (int b = 0; b < RT; ++b) u[a][b] = f32x16{};
    gemm_phase(ys, KBO, u, std::integral_constant<int, FT>{});
    // H = GELU(U) -> hs
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int fl = wave * (HC / 4) + ft * 32 + 16 * g + 8 * hf;   // unit within the chunk
#pragma unroll
        for (int b = 0; b < RT; ++b) {
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = gelu_tanh(u[ft][b][8 * g + e]);
          st_packed(hs + (size_t)((fl >> 4) * RT + b) * kFragElems, lane, v);
        }
      }
    }
    park();
    __syncthreads();
    // Z^T += W_2[:, chunk] H^T
    gemm_phase(hs, KB2, acc, std::integral_constant<int, NT>{});
    __syncthreads();
  }

  // ---- Z = Y + H W_2 (real rows only)
#pragma unroll
  for (int b = 0; b < RT; ++b) {
    const int pos = pos0 + b * 32 + rho;
    if (pos >= N) continue;
    const size_t r = (size_t)seq * N + pos;
#pragma unroll
    for (int a = 0; a < NT; ++a) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = acc[a][b][8 * g + e];
        store8_f32(Z + r * D + n0w + a * 32 + 16 * g + 8 * hf, v);
      }
    }
  }
}

namespace {

template <typename TX, typename T, typename TO, int D, int BM, int P>
int run_ffn(const LayerLaunch& L, hipStream_t s, char* err, size_t n) {
  const size_t smem = (size_t)BM * (D + kFfnChunk) * sizeof(T);
  auto k = ffn_epilogue_kernel<TX, T, TO, D, BM, P>;
  if (set_smem(k, smem, err, n)) return 1;
  // one workgroup per BM packed rows
  hipLaunchKernelGGL(k, dim3(L.batch * L.seq_pad / BM), dim3(256), smem, s, (const TX*)L.x,
                     (const T*)L.q, (const T*)L.wpack + qkv_pack_elems(L.d_model, L.kv_pad),
                     (const T*)L.w.ln2_g, (const T*)L.w.ln2_b, (TO*)L.z, L.seq_len, L.seq_pad,
                     L.d_ff, L.ln_eps);
  return check_launch("ffn_epilogue", err, n);
}

template <typename TX, typename T, typename TO>
int dispatch_ffn(const LayerLaunch& L, hipStream_t s, char* err, size_t n) {
  const int d = L.d_model;
  if constexpr (sizeof(T) == 4) {
    if (d == 128) return run_ffn<TX, T, TO, 128, 64, 2>(L, s, err, n);
    if (d == 256) return run_ffn<TX, T, TO, 256, 32, 2>(L, s, err, n);
  } else {
    if (d == 256) return run_ffn<TX, T, TO, 256, 64, 4>(L, s, err, n);
    if (d == 512) return run_ffn<TX, T, TO, 512, 64, 4>(L, s, err, n);
    if (d == 768) return run_ffn<TX, T, TO, 768, 64, 4>(L, s, err, n);
    if (d == 1024) return run_ffn<TX, T, TO, 1024, 64, 4>(L, s, err, n);
  }
  set_err(err, n, "no epilogue kernel for d_model %s%d", "", d);
  return 1;
}

}  // namespace

int launch_ffn(const LayerLaunch& L, hipStream_t s, char* err, size_t n) {
  if (coop_epilogue(L.d_model, L.split, L.d_ff)) return launch_ffn_coop(L, s, err, n);
  if (staged_epilogue(L.d_model, L.split, L.d_ff)) return launch_ffn_staged(L, s, err, n);
  if (L.compute_f32)
    return L.z_f32 ? dispatch_ffn<float, float, float>(L, s, err, n)
                   : dispatch_ffn<float, float, bf16>(L, s, err, n);
  if (L.x_f32)
    return L.z_f32 ? dispatch_ffn<float, bf16, float>(L, s, err, n)
                   : dispatch_ffn<float, bf16, bf16>(L, s, err, n);
  return L.z_f32 ? dispatch_ffn<bf16, bf16, float>(L, s, err, n)
                 : dispatch_ffn<bf16, bf16, bf16>(L, s, err, n);
}

}  // namespace bpt
