// LN1 into the packed activation operand (gfx950); the QKV projection itself
// is in k_gemm.hip.
//
// "Blockwise Parallel Transformer — BPT" (aicassindra.com), section "The fused
// blockwise algorithm": queries, keys and values are projections of the LN1 rows.
// K and V are projected once for all rows instead of once per inner-loop visit;
// the values are the same.
//
// Rows are handled in "packed row" space: sequence b occupies packed rows
// [b Np, b Np + N) with Np = N rounded up to 128; the padding rows are zero.
// ln_pack: per row, LN1 statistics (mean, biased variance, two passes over the
//   row held in registers) and LN1(x) = (x - mean) / sqrt(var + eps) * g + b,
//   written once in the compute type as matrix-core B fragments (packed order,
//   bpt_device.hpp) -- the projection GEMM's activation operand. The same kernel
//   packs LN2(Y) for the staged epilogue.
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
                                                      T* __restrict__ XP, T* __restrict__ XPlo,
                                                      int B, int N, int Np, int d, float eps) {
  // XPlo (optional): the residual v - bf16(v) of every value, same layout (the lo
  // half of a bf16 pair)
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
  T* outlo = XPlo ? XPlo + (size_t)tile * KS * kFragElems : nullptr;
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
    if (outlo) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] -= bf16_round(v[e]);
      st_packed(outlo + (size_t)ks * kFragElems, lane, v);
    }
  }
}

// 8 consecutive elements of a row as loaded: bf16 rows stay packed (4 registers)
// until the row is normalised; fp32 rows are held as loaded.
template <typename TX>
struct RowChunk;
template <>
struct RowChunk<bf16> {
  uint4 u;
  __device__ void load(const bf16* p) { u = *reinterpret_cast<const uint4*>(p); }
  __device__ void zero() { u = make_uint4(0u, 0u, 0u, 0u); }
  __device__ void widen(float* v) const {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <>
struct RowChunk<float> {
  float f[8];
  __device__ void load(const float* p) { load8_f32(p, f); }
  __device__ void zero() {
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = 0.f;
  }
  __device__ void widen(float* v) const {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = f[e];
  }
};

// LDS-staged variant (d <= 2048): eight waves read a tile's 32 rows once (4 rows
// each, coalesced), normalise them in registers and write the packed fragments
// into LDS; the tile then leaves LDS for global memory as contiguous 16-byte
// chunks. X is read exactly once. Workgroups are persistent over the tiles: as
// soon as a tile is in LDS, the rows of the workgroup's next tile are requested
// into the same registers, so their reads overlap the current tile's writes.
template <typename TX, typename T, int CPL>
__global__ __launch_bounds__(512, (CPL <= 2 && sizeof(TX) == 2) ? 4 : 2) void ln_pack_lds_kernel(const TX* __restrict__ X,
                                                          const T* __restrict__ ln_g,
                                                          const T* __restrict__ ln_b,
                                                          T* __restrict__ XP, int B, int N, int Np,
                                                          int d, float eps, int n_tiles) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* tile_lds = reinterpret_cast<T*>(smem_raw);          // [d/16] packed fragments
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nch = d >> 3;
  int tile = blockIdx.x;
  if (tile >= n_tiles) return;
  // all four rows of this wave are requested before any arithmetic (four rows of
  // loads in flight per wave), and the LN gain and bias once per wave
  RowChunk<TX> raw[4][CPL];
  RowChunk<T> gc[CPL], bc[CPL];
  bool live[4];
  auto load_rows = [&](int t) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = t * 32 + wave + 8 * i;
      const int bi = row / Np, pos = row - bi * Np;
      live[i] = bi < B && pos < N;
      const TX* xr = X + ((size_t)bi * N + pos) * d;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const int c = lane + 64 * j;
        if (live[i] && c < nch) raw[i][j].load(xr + 8 * c);
        else raw[i][j].zero();
      }
    }
  };
  load_rows(tile);
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = lane + 64 * j;
    if (c < nch) {
      gc[j].load(ln_g + 8 * c);
      bc[j].load(ln_b + 8 * c);
    } else {
      gc[j].zero();
      bc[j].zero();
    }
  }
  const int n16 = (32 * d * (int)sizeof(T)) >> 4;         // 16-byte chunks in a tile
  for (;;) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wave + 8 * i;
      float v[CPL][8];
#pragma unroll
      for (int j = 0; j < CPL; ++j) raw[i][j].widen(v[j]);   // chunks past d hold 0
      if (live[i]) {
        float sum = 0.f;
#pragma unroll
        for (int j = 0; j < CPL; ++j)
#pragma unroll
          for (int e = 0; e < 8; ++e) sum += v[j][e];
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
            gc[j].widen(g);
            bc[j].widen(b);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[j][e] = (v[j][e] - mean) * rstd * g[e] + b[e];
          }
        }
      }
      // chunk c (k = 8c .. 8c+7) of row r: fragment c/2, slot 32 (c&1) + pi(r)
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const int c = lane + 64 * j;
        if (c < nch) st_packed(tile_lds + (size_t)(c >> 1) * kFragElems, 32 * (c & 1) + pi_row(r), v[j]);
      }
    }
    __syncthreads();                     // the tile is in LDS; the row registers are free
    const int next = tile + gridDim.x;
    if (next < n_tiles) load_rows(next);
    const uint4* src = reinterpret_cast<const uint4*>(tile_lds);
    uint4* dst = reinterpret_cast<uint4*>(XP + (size_t)tile * 32 * d);
    for (int q = threadIdx.x; q < n16; q += 512) dst[q] = src[q];
    if (next >= n_tiles) break;
    __syncthreads();                     // every wave has copied the tile out of LDS
    tile = next;
  }
}

namespace {

// Persistent grid of the LDS-staged kernel: as many workgroups as the compute units
// hold at once (registers and LDS, as the runtime reports them), or one per tile.
template <typename K>
int ln_grid(K kernel, int n_tiles, size_t smem) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 512, smem) != hipSuccess || per_cu < 1)
    per_cu = 1;
  const int grid = cus * per_cu;
  return n_tiles < grid ? n_tiles : grid;
}

template <typename TX, typename T>
int run_ln_pack(const LayerLaunch& L, hipStream_t s, char* err, size_t n) {
  const int d = L.d_model;
  if (d <= 2048 && !L.split) {
    auto k = d <= 512 ? ln_pack_lds_kernel<TX, T, 1>
                      : (d <= 1024 ? ln_pack_lds_kernel<TX, T, 2> : ln_pack_lds_kernel<TX, T, 4>);
    const size_t smem = (size_t)32 * d * sizeof(T);
    if (set_smem(k, smem, err, n)) return 1;
    const int n_tiles = L.rows_pad / 32;
    hipLaunchKernelGGL(k, dim3(ln_grid(k, n_tiles, smem)), dim3(512), smem, s, (const TX*)L.x,
                       (const T*)L.w.ln1_g, (const T*)L.w.ln1_b, (T*)L.xpack, L.batch, L.seq_len,
                       L.seq_pad, d, L.ln_eps, n_tiles);
    return check_launch("ln_pack", err, n);
  }
  auto k = d <= 1024 ? ln_pack_kernel<TX, T, 2>
                     : (d <= 2048 ? ln_pack_kernel<TX, T, 4> : ln_pack_kernel<TX, T, 8>);
  hipLaunchKernelGGL(k, dim3(L.rows_pad / 32), dim3(256), 0, s, (const TX*)L.x, (const T*)L.w.ln1_g,
                     (const T*)L.w.ln1_b, (T*)L.xpack, (T*)L.xpack_lo, L.batch, L.seq_len, L.seq_pad,
                     d, L.ln_eps);
  return check_launch("ln_pack", err, n);
}

}  // namespace

// phase 0: LN1 into the packed operand; phase 1: the projection GEMM (k_gemm.hip).
int launch_ln_qkv(const LayerLaunch& L, hipStream_t s, char* err, size_t n, int phase) {
  if (phase == 0) {
    if (L.compute_f32) return run_ln_pack<float, float>(L, s, err, n);
    return L.x_f32 ? run_ln_pack<float, bf16>(L, s, err, n) : run_ln_pack<bf16, bf16>(L, s, err, n);
  }
  return launch_qkv(L, s, err, n);
}

// LN2 of the staged epilogue: Y (fp32 [rows, d] over packed rows, row-major)
// into pi-ordered packed fragments in the LN1 operand's buffer.
int launch_ln_rows(const LayerLaunch& L, const void* y, int rows, hipStream_t s, char* err, size_t n) {
  const int d = L.d_model;
  // every packed row is treated as live: sequences of Np rows, Np of them real
  if (d <= 2048 && !L.split) {   // Y read once through LDS (tile [32, d] in bf16)
    auto k = d <= 512 ? ln_pack_lds_kernel<float, bf16, 1>
                      : (d <= 1024 ? ln_pack_lds_kernel<float, bf16, 2> : ln_pack_lds_kernel<float, bf16, 4>);
    const size_t smem = (size_t)32 * d * sizeof(bf16);
    if (set_smem(k, smem, err, n)) return 1;
    hipLaunchKernelGGL(k, dim3(ln_grid(k, rows / 32, smem)), dim3(512), smem, s, (const float*)y,
                       (const bf16*)L.w.ln2_g, (const bf16*)L.w.ln2_b, (bf16*)L.xpack,
                       rows / L.seq_pad, L.seq_pad, L.seq_pad, d, L.ln_eps, rows / 32);
    return check_launch("ln2_rows", err, n);
  }
  auto k = d <= 1024 ? ln_pack_kernel<float, bf16, 2>
                     : (d <= 2048 ? ln_pack_kernel<float, bf16, 4> : ln_pack_kernel<float, bf16, 8>);
  hipLaunchKernelGGL(k, dim3(rows / 32), dim3(256), 0, s, (const float*)y, (const bf16*)L.w.ln2_g,
                     (const bf16*)L.w.ln2_b, (bf16*)L.xpack, (bf16*)L.xpack_lo, rows / L.seq_pad,
                     L.seq_pad, L.seq_pad, d, L.ln_eps);
  return check_launch("ln2_rows", err, n);
}

}  // namespace bpt
