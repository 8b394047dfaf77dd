// Backward pass of the BPT layer (gfx950): the block-recompute backward.
//
// "Blockwise Parallel Transformer — BPT" (aicassindra.com), section "The backward
// pass": the forward keeps the layer input and each row's softmax statistics;
// the backward recomputes the block's scores, attention output and FFN hidden
// state from them and accumulates the gradients of every weight. Here:
//   recompute  LN1(X), Q, K, V (row-major), the attention output A (the attention
//              forward kernel), Y = X + A W_O^T, LN2(Y);
//   FFN        per block of R rows: U = LN2(Y) W_1^T and H = GELU(U) (the block's
//              [R, d_ff] hidden state, never more), dU = (dZ W_2) * GELU'(U),
//              dW_2 += dZ^T H, dW_1 += dU^T LN2(Y), dLN2 = dU W_1;
//   LN2        dY = dZ + LN2 backward of dLN2, and the LN2 gain / bias gradients;
//   W_O        dA = dY W_O, dW_O = dY^T A;
//   attention  dQ, dK, dV from the saved statistic lse (the attention backward);
//   QKV        dLN1 = dQ W_Q + dK W_K + dV W_V, dW_{Q,K,V} = d{Q,K,V}^T LN1(X);
//   LN1        dX = dY + LN1 backward of dLN1, and the LN1 gain / bias gradients.
// Weights are [out, in] row-major, so y = x W^T; gradients come out in the same
// layouts, in fp32. Matrix products take bf16 operands with fp32 accumulation.
//
// Every product runs on one kernel with both operands k-contiguous, C[m, n] =
// sum_k A[m, k] B[n, k] (128 x 128 tiles, k-tiles of 32 staged in LDS through a
// register-prefetched double buffer, v_mfma_f32_32x32x16_bf16, an optional split of
// k over workgroups whose partial sums are added in a fixed order, and epilogues
// that fuse GELU, GELU' and residuals). Operands whose k is their strided index
// (the weights for dX-side products, the activations for the weight gradients,
// which contract over the rows) are first copied transposed by an LDS-tiled
// transpose kernel; the FFN block's U, H and dU are produced transposed ([d_ff,
// rows of the block]) by computing C^T = W x^T, so only dU needs a second layout.
#include <type_traits>

#include "bpt_device.hpp"
#include "bpt_launch.hpp"

namespace bpt {

enum BwdGemmMode {
  kGStoreF32 = 0,   // C = acc (fp32)
  kGAccF32 = 1,     // C += acc (fp32)
  kGStoreBF16 = 2,  // C = bf16(acc)
  kGResid = 3,      // C = R + acc (fp32 out; R fp32 or bf16)
  kGGeluU = 4,      // U = acc (fp32, tile fragment order), H = bf16(GELU(acc))
  kGDGelu = 5,      // C = bf16(acc * GELU'(U)), U as kGGeluU wrote it
  kGPartial = 6     // P[z] = acc (split-k partial sums, fp32)
};

struct BwdGemm {
  const bf16* a;   // A[m, k] at a[m * lda + k]
  const bf16* b;   // B[n, k] at b[n * ldb + k]
  int lda, ldb;    // multiples of 8, like the base pointers' element offsets
  int M, N, K;
  int k_per_split; // multiple of 64; split z covers k in [z kps, (z + 1) kps)
  void* c;         // output (C, H or P)
  int ldc;
  const void* r;   // residual (kGResid)
  int ldr, r_f32;
  // U of kGGeluU (written) and kGDGelu (read), in tile fragment order: per tile
  // (tile row, tile column of the grid), per wave, per 32 x 32 product (i, j), the
  // 16 values of each lane as 4 float4 ([q / 4][lane]); both products have the
  // same M, N and grid, so every lane reads back exactly what it wrote, with
  // 16-byte accesses. ceil(M / 256) * ceil(N / 256) * 65536 floats.
  float* u;
};

// GELU (tanh form) and its derivative: with s = 1 / (1 + exp(-2 z)), z = sqrt(2/pi)
// (u + 0.044715 u^3): GELU(u) = u s, GELU'(u) = s + 2 u s (1 - s) dz/du.
__device__ inline float gelu_tanh_grad(float u) {
  const float k = -2.0f * 0.7978845608028654f * 1.4426950408889634f;
  const float z = u * (1.0f + 0.044715f * u * u);
  const float sg = __builtin_amdgcn_rcpf(1.0f + fast_exp2(k * z));
  const float dz = 0.7978845608028654f * (1.0f + 3.0f * 0.044715f * u * u);
  return sg + 2.0f * u * sg * (1.0f - sg) * dz;
}

namespace {

constexpr int kGBM = 256, kGBN = 256, kGBK = 64;
constexpr int kGStageA = kGBM * kGBK * 2;          // bytes of A per stage (32 KB)
constexpr int kGStage = (kGBM + kGBN) * kGBK * 2;  // bytes per stage (64 KB)
constexpr int kGCopies = kGStage / 1024 / 8;        // 1 KB copies per wave and stage (8)
constexpr int kGCopiesA = kGStageA / 1024 / 8;      // of which A (4)

// LDS layout of a stage: the 16-byte chunk (row r, k-chunk c of 8) of an operand
// tile sits in slot 8 r + (c ^ ((r >> 1) & 7)). The copies write 64 consecutive
// slots per wave instruction (the LDS-DMA path puts lane l at slot base + l), and a
// fragment read (32 consecutive rows, one chunk) hits 16 distinct 16-byte bank
// groups in every 16 lanes.
__device__ inline int chunk_slot(int r, int c) { return 8 * r + (c ^ ((r >> 1) & 7)); }

// Workgroup barrier without a memory fence (__syncthreads() would also wait for
// every copy in flight, including the next k-tile's).
__device__ inline void stage_barrier_bwd() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One k-step's fragments from a stage: A rows at a + 4 KB i (i < 4), B rows at b +
// 4 KB j (j < 2), LDS byte addresses, with the wait for them in the same statement.
// Reads written in C++ would make the compiler wait first for every LDS copy in
// flight (it cannot tell that the copies target other stages).
__device__ inline void ld_frags6(uint32_t a, uint32_t b, bf16x8 (&af)[4], bf16x8 (&bf)[2]) {
  asm volatile(
      "ds_read_b128 %0, %6 offset:0\n\t"
      "ds_read_b128 %1, %6 offset:4096\n\t"
      "ds_read_b128 %2, %6 offset:8192\n\t"
      "ds_read_b128 %3, %6 offset:12288\n\t"
      "ds_read_b128 %4, %7 offset:0\n\t"
      "ds_read_b128 %5, %7 offset:4096\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=v"(af[0]), "=v"(af[1]), "=v"(af[2]), "=v"(af[3]), "=v"(bf[0]), "=v"(bf[1])
      : "v"(a), "v"(b));
}

}  // namespace

// 512 threads = 8 waves in 2 x 4, each 128 x 64 of the 256 x 256 tile (4 x 2
// products of 32 x 32 per k-step: 6 fragment reads from LDS for 8 products). The
// k-tiles (64 wide) are copied global -> LDS by the LDS-DMA path into two 64 KB
// stages, one k-tile ahead of the products (the copy of tile t + 1 is issued once
// tile t has landed), so the loads' latency is covered by a tile of products (four
// k-steps) and no registers stage the data. Rows past M or N read row M - 1 (N - 1),
// and chunks past K read chunk 0: finite values whose products land in discarded
// outputs or are zeroed in the last k-tile's fragments.
template <int MODE>
__global__ __launch_bounds__(512, 1) void bwd_gemm_kernel(BwdGemm g) {
  __shared__ __align__(16) unsigned char st0[kGStage];
  __shared__ __align__(16) unsigned char st1[kGStage];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  // Tile order: workgroups are dealt to the 8 XCDs round-robin; when the tile
  // count divides by 8, XCD x takes a contiguous range of tiles, walked in groups
  // of 4 M-tiles across N, so the tiles an XCD runs together share operand rows in
  // its L2.
  int tm = blockIdx.y, tn = blockIdx.x;
  {
    const int gx = gridDim.x, gy = gridDim.y, T = gx * gy, id = blockIdx.x + gx * blockIdx.y;
    if ((T & 7) == 0 && (gy & 3) == 0) {
      const int t = (id & 7) * (T >> 3) + (id >> 3);
      const int grp = t / (4 * gx), w = t - grp * 4 * gx;
      tm = grp * 4 + (w & 3);
      tn = w >> 2;
    }
  }
  const int m0 = tm * kGBM, n0 = tn * kGBN;
  const int kb = blockIdx.z * g.k_per_split;
  const int ke = min(g.K, kb + g.k_per_split);
  const int nkt = ke > kb ? (ke - kb + kGBK - 1) / kGBK : 0;

  // this wave's copies: A instructions [4 wave, 4 wave + 4), B [2 wave, 2 wave + 2);
  // per copy the source row and k-chunk of this lane (fixed over the k-tiles)
  const bf16* src[kGCopies];
  int ck[kGCopies];
#pragma unroll
  for (int q = 0; q < kGCopies; ++q) {
    const bool isa = q < kGCopiesA;
    const int slot = (isa ? kGCopiesA * wave + q : kGCopiesA * wave + (q - kGCopiesA)) * 64 + lane;
    const int r = slot >> 3, c = (slot & 7) ^ ((r >> 1) & 7);
    const int rows = isa ? g.M : g.N, r0 = isa ? m0 : n0;
    const int gr = min(r0 + r, rows - 1);
    src[q] = (isa ? g.a + (size_t)gr * g.lda : g.b + (size_t)gr * g.ldb);
    ck[q] = 8 * c;
  }
  auto issue = [&](int t, unsigned char* st) __attribute__((always_inline)) {
    const int k0 = kb + t * kGBK;
#pragma unroll
    for (int q = 0; q < kGCopies; ++q) {
      const int gk = k0 + ck[q] < ke ? k0 + ck[q] : 0;
      unsigned char* dst = st + (q < kGCopiesA ? (kGCopiesA * wave + q) * 1024
                                               : kGStageA + (kGCopiesA * wave + (q - kGCopiesA)) * 1024);
      dma16(src[q] + gk, dst);
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  // byte offsets within a stage of this lane's fragment rows for k-step ks: row r
  // = 32 q + (lane & 31) (q a multiple of 32 rows) sits at 128 r + 16 (c ^ ((r >> 1)
  // & 7)), c = 2 ks + lane / 32, and (r >> 1) & 7 depends on the lane only
  uint32_t lofs[kGBK / 16];
#pragma unroll
  for (int ks = 0; ks < kGBK / 16; ++ks)
    lofs[ks] = 128u * (uint32_t)(lane & 31) + 16u * (uint32_t)((2 * ks + (lane >> 5)) ^ ((lane >> 1) & 7));
  const uint32_t aofs = 128u * 128u * (uint32_t)wm, bofs = (uint32_t)kGStageA + 128u * 64u * (uint32_t)wn;
  // fragments of k-step ks from stage st (C++ reads: the stages are separate arrays
  // chosen at compile time, so the compiler does not wait for the copy into the
  // other stage before them), the next k-step's read while this one's products run
  auto frags = [&](const unsigned char* st, int ks, bf16x8 (&af)[4], bf16x8 (&bf)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = *reinterpret_cast<const bf16x8*>(st + aofs + lofs[ks] + 4096 * i);
#pragma unroll
    for (int j = 0; j < 2; ++j) bf[j] = *reinterpret_cast<const bf16x8*>(st + bofs + lofs[ks] + 4096 * j);
  };
  auto compute = [&](int t, const unsigned char* st) __attribute__((always_inline)) {
    const int k0 = kb + t * kGBK;
    const bool edge = k0 + kGBK > ke;   // the last k-tile runs past K
    bf16x8 af[2][4], bfr[2][2];
    frags(st, 0, af[0], bfr[0]);
#pragma unroll
    for (int ks = 0; ks < kGBK / 16; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < kGBK / 16) frags(st, ks + 1, af[cur ^ 1], bfr[cur ^ 1]);
      if (edge) {
        const int c = 2 * ks + (lane >> 5);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (k0 + 8 * c + e >= ke) {
#pragma unroll
            for (int i = 0; i < 4; ++i) af[cur][i][e] = (bf16)0.0f;
#pragma unroll
            for (int j = 0; j < 2; ++j) bfr[cur][j][e] = (bf16)0.0f;
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][i], bfr[cur][j], acc[i][j], 0, 0, 0);
    }
  };

  if (nkt > 0) issue(0, st0);
  // step t: wait for this wave's copies of tile t, barrier (every wave's copies of t
  // landed; every wave is done with t - 1, whose stage takes t + 1), issue t + 1,
  // multiply t
  auto step = [&](int t, const unsigned char* rd, unsigned char* wr) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0070);
    stage_barrier_bwd();
    if (t + 1 < nkt) issue(t + 1, wr);
    compute(t, rd);
  };
  for (int t = 0; t < nkt; t += 2) {
    step(t, st0, st1);
    if (t + 1 < nkt) step(t + 1, st1, st0);
  }

  // C layout: lane l holds column l % 32; register q holds row 8 (q / 4) + 4 (l / 32) + q % 4
  float* const ut = (MODE == kGGeluU || MODE == kGDGelu)
                        ? g.u + ((((size_t)tm * gridDim.x + tn) * 8 + wave) << 13)   // 8192 floats per wave
                        : nullptr;
  // kGDGelu: U of product (i, j) is loaded one product ahead, before the stores of
  // the current one (which the compiler would not move the loads across)
  float4 unext[4];
  auto load_u = [&](int ij) __attribute__((always_inline)) {
    const float4* up = reinterpret_cast<const float4*>(ut + (ij << 10)) + lane;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) unext[q4] = up[q4 * 64];
  };
  if constexpr (MODE == kGDGelu) load_u(0);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float uv[16];
      if constexpr (MODE == kGGeluU) {
        float4* up = reinterpret_cast<float4*>(ut + ((i * 2 + j) << 10)) + lane;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          up[q4 * 64] = make_float4(acc[i][j][4 * q4], acc[i][j][4 * q4 + 1], acc[i][j][4 * q4 + 2],
                                    acc[i][j][4 * q4 + 3]);
      } else if constexpr (MODE == kGDGelu) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          uv[4 * q4] = unext[q4].x;
          uv[4 * q4 + 1] = unext[q4].y;
          uv[4 * q4 + 2] = unext[q4].z;
          uv[4 * q4 + 3] = unext[q4].w;
        }
        if (i * 2 + j + 1 < 8) load_u(i * 2 + j + 1);
      }
      const int n = n0 + wn * 64 + j * 32 + (lane & 31);
      if (n >= g.N) continue;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int m = m0 + wm * 128 + i * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
        if (m >= g.M) continue;
        const float v = acc[i][j][q];
        const size_t o = (size_t)m * g.ldc + n;
        if constexpr (MODE == kGStoreF32) {
          static_cast<float*>(g.c)[o] = v;
        } else if constexpr (MODE == kGAccF32) {
          static_cast<float*>(g.c)[o] += v;
        } else if constexpr (MODE == kGStoreBF16) {
          static_cast<bf16*>(g.c)[o] = (bf16)v;
        } else if constexpr (MODE == kGResid) {
          const size_t ro = (size_t)m * g.ldr + n;
          const float r = g.r_f32 ? static_cast<const float*>(g.r)[ro] : (float)static_cast<const bf16*>(g.r)[ro];
          static_cast<float*>(g.c)[o] = r + v;
        } else if constexpr (MODE == kGGeluU) {
          static_cast<bf16*>(g.c)[o] = (bf16)gelu_tanh(v);
        } else if constexpr (MODE == kGDGelu) {
          static_cast<bf16*>(g.c)[o] = (bf16)(v * gelu_tanh_grad(uv[q]));
        } else {   // kGPartial
          static_cast<float*>(g.c)[(size_t)blockIdx.z * g.M * g.N + (size_t)m * g.N + n] = v;
        }
      }
    }
}

// C (fp32 [M, N], ldc) = [C +] sum over z of P[z] (the split-k partials, in order).
__global__ __launch_bounds__(256) void bwd_reduce_kernel(float* c, int ldc, const float* p, int M, int N,
                                                         int splits, int accumulate) {
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= (long long)M * N) return;
  const int m = (int)(t / N), n = (int)(t % N);
  float s = accumulate ? c[(size_t)m * ldc + n] : 0.f;
  for (int z = 0; z < splits; ++z) s += p[(size_t)z * M * N + t];
  c[(size_t)m * ldc + n] = s;
}

// LN of each row (one wave per row, d <= 4096): out = bf16(LN(x) g + b), stats =
// (mean, rstd).
template <typename TX>
__global__ __launch_bounds__(256) void bwd_ln_fwd_kernel(const TX* __restrict__ x, const bf16* __restrict__ gain,
                                                         const bf16* __restrict__ bias, bf16* __restrict__ out,
                                                         float2* __restrict__ stats, int rows, int d, float eps) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const TX* xr = x + (size_t)row * d;
  float s = 0.f;
  for (int c = lane * 8; c < d; c += 512) {
    float v[8];
    load8_f32(xr + c, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) s += v[e];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
  const float mean = s / d;
  float q = 0.f;
  for (int c = lane * 8; c < d; c += 512) {
    float v[8];
    load8_f32(xr + c, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) q += (v[e] - mean) * (v[e] - mean);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) q += __shfl_xor(q, o, 64);
  const float rstd = 1.0f / sqrtf(q / d + eps);
  for (int c = lane * 8; c < d; c += 512) {
    float v[8], gv[8], bv[8];
    load8_f32(xr + c, v);
    load8_f32(gain + c, gv);
    load8_f32(bias + c, bv);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (v[e] - mean) * rstd * gv[e] + bv[e];
    store8_f32(out + (size_t)row * d + c, v);
  }
  if (lane == 0) stats[row] = make_float2(mean, rstd);
}

// LN backward of each row: out = resid + rstd (g - mean(g) - xh mean(g xh)),
// g = dy * gain, xh = (x - mean) rstd; optionally a bf16 copy of out. Column
// sums of dy xh and dy over the workgroup's rows go to part[blockIdx][2][d]
// (summed in a fixed order afterwards). One wave per row, rows strided over the
// workgroups; d <= 4096 (8 slabs of 512 columns, 8 per lane).
template <typename TX>
__global__ __launch_bounds__(256) void bwd_ln_bwd_kernel(const TX* __restrict__ x, const float2* __restrict__ stats,
                                                         const bf16* __restrict__ gain, const float* __restrict__ dy,
                                                         const float* __restrict__ resid, float* __restrict__ out,
                                                         bf16* __restrict__ out_bf16, float* __restrict__ part,
                                                         int rows, int d) {
  __shared__ float red[4][2][512];     // per wave column partials of one 512-column slab
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float cg[8][8], cb[8][8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) cg[j][e] = cb[j][e] = 0.f;
  for (int row = blockIdx.x * 4 + wave; row < rows; row += gridDim.x * 4) {
    const float2 st = stats[row];
    const TX* xr = x + (size_t)row * d;
    const float* dr = dy + (size_t)row * d;
    float sg = 0.f, sgx = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = lane * 8 + 512 * j;
      if (c < d) {
        float xv[8], dv[8], gv[8];
        load8_f32(xr + c, xv);
        load8_f32(dr + c, dv);
        load8_f32(gain + c, gv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float xh = (xv[e] - st.x) * st.y, gg = dv[e] * gv[e];
          sg += gg;
          sgx += gg * xh;
          cg[j][e] += dv[e] * xh;
          cb[j][e] += dv[e];
        }
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      sg += __shfl_xor(sg, o, 64);
      sgx += __shfl_xor(sgx, o, 64);
    }
    sg /= d;
    sgx /= d;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = lane * 8 + 512 * j;
      if (c < d) {
        float xv[8], dv[8], gv[8], rv[8], o8[8];
        load8_f32(xr + c, xv);
        load8_f32(dr + c, dv);
        load8_f32(gain + c, gv);
        load8_f32(resid + (size_t)row * d + c, rv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float xh = (xv[e] - st.x) * st.y;
          o8[e] = rv[e] + st.y * (dv[e] * gv[e] - sg - xh * sgx);
        }
        store8_f32(out + (size_t)row * d + c, o8);
        if (out_bf16) store8_f32(out_bf16 + (size_t)row * d + c, o8);
      }
    }
  }
  // column partials: the four waves combine through LDS, slab by slab
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (512 * j >= d) break;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      red[wave][0][lane * 8 + e] = cg[j][e];
      red[wave][1][lane * 8 + e] = cb[j][e];
    }
    __syncthreads();
    for (int c = threadIdx.x; c < 512; c += 256) {
      const int col = 512 * j + c;
      if (col < d) {
        part[((size_t)blockIdx.x * 2 + 0) * d + col] = red[0][0][c] + red[1][0][c] + red[2][0][c] + red[3][0][c];
        part[((size_t)blockIdx.x * 2 + 1) * d + col] = red[0][1][c] + red[1][1][c] + red[2][1][c] + red[3][1][c];
      }
    }
    __syncthreads();
  }
}

// dgain[c], dbias[c] = sum over the workgroups' partials: 32 columns per workgroup,
// 8 slices per column (parts s, s + 8, ...), each added in order, then the 8 slice
// sums in order (a fixed order, so results repeat bit for bit).
__global__ __launch_bounds__(256) void bwd_colsum_kernel(const float* __restrict__ part, int nparts, int d,
                                                         float* __restrict__ dgain, float* __restrict__ dbias) {
  __shared__ float red[2][8][32];
  const int cl = threadIdx.x & 31, sl = threadIdx.x >> 5;
  const int c = blockIdx.x * 32 + cl;
  float sg = 0.f, sb = 0.f;
  if (c < d) {
    for (int p = sl; p < nparts; p += 8) {
      sg += part[((size_t)p * 2 + 0) * d + c];
      sb += part[((size_t)p * 2 + 1) * d + c];
    }
  }
  red[0][sl][cl] = sg;
  red[1][sl][cl] = sb;
  __syncthreads();
  if (sl == 0 && c < d) {
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      a += red[0][k][cl];
      b += red[1][k][cl];
    }
    dgain[c] = a;
    dbias[c] = b;
  }
}

// out[c, r] = in[r, c] (bf16 out; ld_out >= nr) for in [nr, nc] with row stride
// ld_in, through a 64 x 64 LDS tile. With out_rm, also a bf16 row-major copy of in
// (row stride ld_rm), for fp32 inputs. Global accesses are 8 elements per lane
// (16 bytes of bf16) where the strides and base addresses allow (vec_in: in and
// out_rm; vec_out: out), else element by element; the tile's row pitch of 65
// elements keeps the column reads of the second phase on distinct LDS banks.
template <typename TIn>
__global__ __launch_bounds__(256) void bwd_transpose_kernel(const TIn* __restrict__ in, int nr, int nc, int ld_in,
                                                            bf16* __restrict__ out, int ld_out,
                                                            bf16* __restrict__ out_rm, int ld_rm, int vec_in,
                                                            int vec_out) {
  constexpr int P = 65;
  __shared__ bf16 tile[64 * P];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;   // rows on x: up to 2^31 - 1 blocks
  const int sub = threadIdx.x & 7, rr = threadIdx.x >> 3;
  // phase 1: rows rr, rr + 32 of the tile, columns 8 sub .. 8 sub + 7
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int r = rr + 32 * p, gr = r0 + r, gc = c0 + 8 * sub;
    float v[8];
    const bool full = gr < nr && gc + 8 <= nc;
    if (full && vec_in) {
      load8_f32(in + (size_t)gr * ld_in + gc, v);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        v[e] = (gr < nr && gc + e < nc) ? (float)in[(size_t)gr * ld_in + gc + e] : 0.f;
    }
    if (out_rm != nullptr) {
      if (full && vec_in) {
        store8_f32(out_rm + (size_t)gr * ld_rm + gc, v);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (gr < nr && gc + e < nc) out_rm[(size_t)gr * ld_rm + gc + e] = (bf16)v[e];
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[r * P + 8 * sub + e] = (bf16)v[e];
  }
  __syncthreads();
  // phase 2: output rows (input columns) rr, rr + 32, input rows 8 sub .. 8 sub + 7
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int c = rr + 32 * p, gc = c0 + c, gr = r0 + 8 * sub;
    if (gc >= nc) continue;
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (float)tile[(8 * sub + j) * P + c];
    bf16* o = out + (size_t)gc * ld_out + gr;
    if (gr + 8 <= nr && vec_out) {
      store8_f32(o, v);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (gr + j < nr) o[j] = (bf16)v[j];
    }
  }
}

namespace {

template <int MODE>
int run_bwd_gemm(const BwdGemm& g0, int splits, hipStream_t s, const char* what, char* err, size_t n) {
  BwdGemm g = g0;
  if (g.M <= 0 || g.N <= 0) return 0;
  if (splits < 1) splits = 1;
  g.k_per_split = ((g.K + splits - 1) / splits + kGBK - 1) / kGBK * kGBK;
  if (g.k_per_split < kGBK) g.k_per_split = kGBK;
  splits = (g.K + g.k_per_split - 1) / g.k_per_split;
  if (splits < 1) splits = 1;
  dim3 grid((g.N + kGBN - 1) / kGBN, (g.M + kGBM - 1) / kGBM, splits);
  if (grid.y > 65535 || grid.z > 65535) {
    set_err(err, n, "%s: product too tall for the grid", what);
    return 1;
  }
  hipLaunchKernelGGL((bwd_gemm_kernel<MODE>), grid, dim3(512), 0, s, g);
  return check_launch(what, err, n);
}

// C (+)= A B^T with k split over `splits` workgroup layers into the partial
// buffer, then reduced in order into C.
int run_bwd_gemm_split(BwdGemm g, int splits, float* partials, bool accumulate, hipStream_t s,
                       const char* what, char* err, size_t n) {
  if (splits <= 1)
    return accumulate ? run_bwd_gemm<kGAccF32>(g, 1, s, what, err, n)
                      : run_bwd_gemm<kGStoreF32>(g, 1, s, what, err, n);
  float* c = static_cast<float*>(g.c);
  const int ldc = g.ldc;
  g.c = partials;
  int kps = ((g.K + splits - 1) / splits + kGBK - 1) / kGBK * kGBK;
  if (kps < kGBK) kps = kGBK;
  const int used = (g.K + kps - 1) / kps;
  if (run_bwd_gemm<kGPartial>(g, splits, s, what, err, n)) return 1;
  const long long mn = (long long)g.M * g.N;
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)((mn + 255) / 256)), dim3(256), 0, s, c, ldc, partials,
                     g.M, g.N, used, accumulate ? 1 : 0);
  return check_launch("bwd_reduce", err, n);
}

template <typename TIn>
int transpose(const TIn* in, int nr, int nc, int ld_in, bf16* out, int ld_out, bf16* out_rm, hipStream_t s,
              char* err, size_t n, int ld_rm = 0) {
  if (nr <= 0 || nc <= 0) return 0;
  if ((nc + 63) / 64 > 65535) {
    set_err(err, n, "bwd_transpose: too many columns%s (%d)", "", nc);
    return 1;
  }
  if (!ld_rm) ld_rm = ld_in;
  auto a16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  const int vec_in = (ld_in % 8 == 0) && a16(in) && (out_rm == nullptr || ((ld_rm % 8 == 0) && a16(out_rm)));
  const int vec_out = (ld_out % 8 == 0) && a16(out);
  hipLaunchKernelGGL(bwd_transpose_kernel<TIn>, dim3((nr + 63) / 64, (nc + 63) / 64), dim3(256), 0, s, in, nr, nc,
                     ld_in, out, ld_out, out_rm, ld_rm, vec_in, vec_out);
  return check_launch("bwd_transpose", err, n);
}

template <typename TX>
int ln_bwd(const TX* x, const float2* stats, const bf16* gain, const float* dy, const float* resid, float* out,
           bf16* out_bf16, float* part, int nparts, float* dgain, float* dbias, int rows, int d, hipStream_t s,
           char* err, size_t n) {
  hipLaunchKernelGGL(bwd_ln_bwd_kernel<TX>, dim3(nparts), dim3(256), 0, s, x, stats, gain, dy, resid, out, out_bf16,
                     part, rows, d);
  if (check_launch("bwd_ln_bwd", err, n)) return 1;
  hipLaunchKernelGGL(bwd_colsum_kernel, dim3((d + 31) / 32), dim3(256), 0, s, part, nparts, d, dgain, dbias);
  return check_launch("bwd_colsum", err, n);
}

}  // namespace

int launch_layer_bwd(const LayerBwdLaunch& L, void* stream, char* err, size_t n) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int rows = L.rows, d = L.d_model, f = L.d_ff, rt = L.rows_t, bl = L.blk_ld;
  // K and V are [rows, dkv] with n_kv_heads key/value heads; [dQ dK dV] and the stacked
  // transposed W_Q, W_K, W_V are k3 = d + 2 dkv wide
  const int G = L.n_kv_heads > 0 ? L.n_kv_heads : L.n_heads, dkv = G * (d / L.n_heads), k3 = d + 2 * dkv;
  if (d % 64 != 0 || d > 4096 || f % 256 != 0 || L.block_rows < 1 || L.ln_parts < 1 || rt < rows ||
      L.n_heads % G != 0 || dkv % 64 != 0 ||
      rt % 8 != 0 || bl < L.block_rows || bl % 8 != 0 || (L.block_rows < rows && L.block_rows % 8 != 0)) {
    set_err(err, n, "layer backward: inconsistent launch shape%s (d_model %d)", "", d);
    return 1;
  }
  auto B = [](void* p) { return static_cast<bf16*>(p); };
  auto CB = [](const void* p) { return static_cast<const bf16*>(p); };
  const bf16* const x = CB(L.x);
  const bf16* const wq = CB(L.w.w_q);
  const bf16* const wk = CB(L.w.w_k);
  const bf16* const wv = CB(L.w.w_v);
  const bf16* const wo = CB(L.w.w_o);
  const bf16* const w1 = CB(L.w.w_1);
  const bf16* const w2 = CB(L.w.w_2);
  bf16 *const x1 = B(L.x1), *const q = B(L.q), *const k = B(L.k), *const v = B(L.v);
  bf16 *const attn = B(L.attn), *const y2 = B(L.y2), *const dzb = B(L.dzb), *const dyb = B(L.dyb);
  bf16 *const x1t = B(L.x1t), *const attnt = B(L.attnt), *const y2t = B(L.y2t), *const dzt = B(L.dzt);
  bf16 *const dyt = B(L.dyt), *const da = B(L.da);
  bf16 *const hblk = B(L.hblk), *const dublk = B(L.dublk), *const dub = B(L.dub);
  bf16 *const w1t = B(L.w1t), *const w2t = B(L.w2t), *const wot = B(L.wot);
  bf16* const wqkvt = B(L.wqkvt);   // [d, k3]: W_Q^T | W_K^T | W_V^T
  bf16* const dqkvb = B(L.dqkvb);   // [rows, k3]: dQ | dK | dV in bf16
  bf16* const dqkvt[3] = {B(L.dqt), B(L.dkt), B(L.dvt)};
  float2* const stats1 = reinterpret_cast<float2*>(L.stats1);
  float2* const stats2 = reinterpret_cast<float2*>(L.stats2);
  const int wsplit = L.wgrad_splits;

  // ---- the weights with their input index contiguous ([in, out]), for dX-side products
  if (transpose(w1, f, d, d, w1t, f, nullptr, s, err, n) || transpose(w2, d, f, f, w2t, d, nullptr, s, err, n) ||
      transpose(wo, d, d, d, wot, d, nullptr, s, err, n) || transpose(wq, d, d, d, wqkvt, k3, nullptr, s, err, n) ||
      transpose(wk, dkv, d, d, wqkvt + d, k3, nullptr, s, err, n) ||
      transpose(wv, dkv, d, d, wqkvt + d + dkv, k3, nullptr, s, err, n))
    return 1;

  // ---- recompute: LN1(X), Q, K, V, A, Y = X + A W_O^T, LN2(Y); transposed copies of
  //      LN1(X), A, LN2(Y) and dZ for the weight gradients
  hipLaunchKernelGGL(bwd_ln_fwd_kernel<bf16>, dim3((rows + 3) / 4), dim3(256), 0, s, x, CB(L.w.ln1_g),
                     CB(L.w.ln1_b), x1, stats1, rows, d, L.ln_eps);
  if (check_launch("bwd_ln1", err, n)) return 1;
  if (transpose(x1, rows, d, d, x1t, rt, nullptr, s, err, n)) return 1;
  {
    const bf16* ws[3] = {wq, wk, wv};
    bf16* outs[3] = {q, k, v};
    for (int i = 0; i < 3; ++i) {
      const int w = i == 0 ? d : dkv;
      BwdGemm g{};
      g.a = x1; g.lda = d; g.b = ws[i]; g.ldb = d; g.M = rows; g.N = w; g.K = d; g.c = outs[i]; g.ldc = w;
      if (run_bwd_gemm<kGStoreBF16>(g, 1, s, "bwd_qkv", err, n)) return 1;
    }
  }
  {
    AttnFwdLaunch a{};
    a.batch = L.batch; a.seq_len = L.seq_len; a.seq_pad = L.seq_pad; a.d_model = d;
    a.n_heads = L.n_heads; a.d_head = d / L.n_heads; a.causal = L.causal;
    a.n_kv_heads = G; a.window = L.window; a.chunk = L.chunk;
    a.q = q; a.k = k; a.v = v; a.o = attn; a.lse = L.lse_re;
    for (int i = 0; i < 3; ++i) a.packed[i] = L.packed[i];
    if (launch_attention_fwd(a, stream, err, n)) return 1;
  }
  if (transpose(attn, rows, d, d, attnt, rt, nullptr, s, err, n)) return 1;
  {
    BwdGemm g{};
    g.a = attn; g.lda = d; g.b = wo; g.ldb = d; g.M = rows; g.N = d; g.K = d;
    g.c = L.y; g.ldc = d; g.r = x; g.ldr = d; g.r_f32 = 0;
    if (run_bwd_gemm<kGResid>(g, 1, s, "bwd_wo_fwd", err, n)) return 1;
  }
  hipLaunchKernelGGL(bwd_ln_fwd_kernel<float>, dim3((rows + 3) / 4), dim3(256), 0, s, L.y, CB(L.w.ln2_g),
                     CB(L.w.ln2_b), y2, stats2, rows, d, L.ln_eps);
  if (check_launch("bwd_ln2", err, n)) return 1;
  if (transpose(y2, rows, d, d, y2t, rt, nullptr, s, err, n)) return 1;
  if (transpose(L.dz, rows, d, d, dzt, rt, dzb, s, err, n)) return 1;   // also dZ in bf16, row-major

  // ---- FFN, one block of at most block_rows rows at a time; the block's U, H, dU
  //      are [d_ff, R] (row stride blk_ld), dU also [R, d_ff]
  for (int r0 = 0; r0 < rows; r0 += L.block_rows) {
    const int R = rows - r0 < L.block_rows ? rows - r0 : L.block_rows;
    BwdGemm g{};
    // U^T = W_1 LN2(Y)^T, H^T = GELU(U^T)
    g.a = w1; g.lda = d; g.b = y2 + (size_t)r0 * d; g.ldb = d; g.M = f; g.N = R; g.K = d;
    g.c = hblk; g.ldc = bl; g.u = L.ublk;
    if (run_bwd_gemm<kGGeluU>(g, 1, s, "bwd_w1_fwd", err, n)) return 1;
    // dU^T = (W_2^T dZ^T) * GELU'(U^T): W_2^T is [d_ff, d]
    g = BwdGemm{};
    g.a = w2t; g.lda = d; g.b = dzb + (size_t)r0 * d; g.ldb = d; g.M = f; g.N = R; g.K = d;
    g.c = dublk; g.ldc = bl; g.u = L.ublk;
    if (run_bwd_gemm<kGDGelu>(g, 1, s, "bwd_du", err, n)) return 1;
    if (transpose(dublk, f, R, bl, dub, f, nullptr, s, err, n)) return 1;
    // dW_2 (+)= dZ^T H: A = dZ^T [d, rows] (columns of the block), B = H^T [d_ff, R]
    g = BwdGemm{};
    g.a = dzt + r0; g.lda = rt; g.b = hblk; g.ldb = bl; g.M = d; g.N = f; g.K = R;
    g.c = L.g.w_2; g.ldc = f;
    if (run_bwd_gemm_split(g, L.ffn_splits, L.partials, r0 > 0, s, "bwd_dw2", err, n)) return 1;
    // dW_1 (+)= dU^T LN2(Y): A = dU^T [d_ff, R], B = LN2(Y)^T [d, rows]
    g = BwdGemm{};
    g.a = dublk; g.lda = bl; g.b = y2t + r0; g.ldb = rt; g.M = f; g.N = d; g.K = R;
    g.c = L.g.w_1; g.ldc = d;
    if (run_bwd_gemm_split(g, L.ffn_splits, L.partials, r0 > 0, s, "bwd_dw1", err, n)) return 1;
    // dLN2 = dU W_1: A = dU [R, d_ff], B = W_1^T [d, d_ff]
    g = BwdGemm{};
    g.a = dub; g.lda = f; g.b = w1t; g.ldb = f; g.M = R; g.N = d; g.K = f;
    g.c = L.dy2 + (size_t)r0 * d; g.ldc = d;
    if (run_bwd_gemm<kGStoreF32>(g, 1, s, "bwd_dln2", err, n)) return 1;
  }
  // ---- LN2 backward: dY = dZ + LN2'(dLN2) (and a bf16 copy); LN2 gain / bias gradients
  if (ln_bwd<float>(L.y, stats2, CB(L.w.ln2_g), L.dy2, L.dz, L.dy, dyb, L.ln_part, L.ln_parts, L.g.ln2_g,
                    L.g.ln2_b, rows, d, s, err, n))
    return 1;
  if (transpose(dyb, rows, d, d, dyt, rt, nullptr, s, err, n)) return 1;
  // ---- W_O: dA = dY W_O, dW_O = dY^T A
  {
    BwdGemm g{};
    g.a = dyb; g.lda = d; g.b = wot; g.ldb = d; g.M = rows; g.N = d; g.K = d; g.c = da; g.ldc = d;
    if (run_bwd_gemm<kGStoreBF16>(g, 1, s, "bwd_da", err, n)) return 1;
    g = BwdGemm{};
    g.a = dyt; g.lda = rt; g.b = attnt; g.ldb = rt; g.M = d; g.N = d; g.K = rows; g.c = L.g.w_o; g.ldc = d;
    if (run_bwd_gemm_split(g, wsplit, L.partials, false, s, "bwd_dwo", err, n)) return 1;
  }
  // ---- attention backward from the saved statistic
  {
    AttnBwdLaunch a{};
    a.batch = L.batch; a.seq_len = L.seq_len; a.d_model = d; a.n_heads = L.n_heads;
    a.d_head = d / L.n_heads; a.causal = L.causal; a.n_kv_heads = G; a.window = L.window; a.chunk = L.chunk;
    a.seq_pad = L.seq_pad;
    a.q = q; a.k = k; a.v = v; a.out = attn; a.dout = da; a.lse = L.lse;
    a.dq = L.dq; a.dk = L.dk; a.dv = L.dv;
    a.stat_d = L.stat_d; a.stat_l2 = L.stat_l2;
    for (int i = 0; i < kAttnBwdPacked; ++i) a.packed[i] = L.packed[i];
    if (launch_attention_bwd(a, stream, err, n)) return 1;
  }
  // ---- QKV: dLN1 = [dQ dK dV] [W_Q; W_K; W_V] (one product over k3), dW_{Q,K,V} = d{Q,K,V}^T LN1(X)
  {
    const float* dg[3] = {L.dq, L.dk, L.dv};
    float* dw[3] = {L.g.w_q, L.g.w_k, L.g.w_v};
    const int width[3] = {d, dkv, dkv}, col[3] = {0, d, d + dkv};
    for (int i = 0; i < 3; ++i) {
      if (transpose(dg[i], rows, width[i], width[i], dqkvt[i], rt, dqkvb + col[i], s, err, n, k3)) return 1;
      BwdGemm g{};
      g.a = dqkvt[i]; g.lda = rt; g.b = x1t; g.ldb = rt; g.M = width[i]; g.N = d; g.K = rows; g.c = dw[i];
      g.ldc = d;
      if (run_bwd_gemm_split(g, wsplit, L.partials, false, s, "bwd_dwqkv", err, n)) return 1;
    }
    BwdGemm g{};
    g.a = dqkvb; g.lda = k3; g.b = wqkvt; g.ldb = k3; g.M = rows; g.N = d; g.K = k3; g.c = L.dx1; g.ldc = d;
    if (run_bwd_gemm<kGStoreF32>(g, 1, s, "bwd_dx1", err, n)) return 1;
  }
  // ---- LN1 backward: dX = dY + LN1'(dLN1); LN1 gain / bias gradients
  return ln_bwd<bf16>(x, stats1, CB(L.w.ln1_g), L.dx1, L.dy, L.dx, nullptr, L.ln_part, L.ln_parts, L.g.ln1_g,
                      L.g.ln1_b, rows, d, s, err, n);
}

}  // namespace bpt
