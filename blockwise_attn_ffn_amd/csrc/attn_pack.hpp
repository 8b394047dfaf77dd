// Copies of row-major attention operands [batch * N, d] (bf16, heads concatenated)
// into the matrix-core fragment layouts the attention kernels read
// (bpt_device.hpp: packed fragments), zero past N in each sequence's Np rows:
//   rows-B: B fragments over [token rows, d], rows in natural order (Q, and O back)
//   rows-A: per (sequence, head) A fragments over [tokens (pi order), d_k]   (K)
//   cols-A: per (sequence, head) A fragments over [d_k (pi order), tokens]   (V^T)
// The kernels are local to each translation unit that includes this header.
#pragma once

#include "bpt_device.hpp"

namespace bpt {
namespace {

// Transpose into cols-A fragments. One workgroup per (tensor, sequence, head,
// 64-token tile, 64-feature tile): the tile is read row by row (coalesced) into
// LDS, then written as 8 whole fragments (2 feature tiles of 32 x 4 token k-steps).
struct TransposeJob {
  const bf16* src[3];
  bf16* dst[3];
};

__global__ __launch_bounds__(256) void bwd_transpose_kernel(TransposeJob job, int N, int Np, int H,
                                                            int dk) {
  __shared__ __align__(16) bf16 tile[64][72];     // [token][feature], rows padded to 144 B
  const bf16* __restrict__ src = job.src[blockIdx.y];
  bf16* __restrict__ dst = job.dst[blockIdx.y];
  const int d = H * dk, ftiles = dk / 64, ttiles = Np / 64;
  int x = blockIdx.x;
  const int ft = x % ftiles;
  x /= ftiles;
  const int tt = x % ttiles;
  const int bh = x / ttiles;
  const int b = bh / H, h = bh - b * H;
#pragma unroll
  for (int i = threadIdx.x; i < 512; i += 256) {
    const int r = i >> 3, c = i & 7, pos = tt * 64 + r;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (pos < N)
      v = *reinterpret_cast<const uint4*>(src + ((size_t)b * N + pos) * d + (size_t)h * dk + ft * 64 + c * 8);
    *reinterpret_cast<uint4*>(&tile[r][c * 8]) = v;
  }
  __syncthreads();
#pragma unroll
  for (int i = threadIdx.x; i < 512; i += 256) {
    const int f = i >> 6, slot = i & 63;
    const int dtl = f >> 2, ks = f & 3;
    const int feat = dtl * 32 + pi_row(slot & 31), tok0 = ks * 16 + 8 * (slot >> 5);
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = tile[tok0 + e][feat];
    const size_t frag = ((size_t)bh * (dk / 32) + ft * 2 + dtl) * (Np / 16) + tt * 4 + ks;
    *reinterpret_cast<bf16x8*>(dst + frag * kFragElems + slot * 8) = v;
  }
}


enum RowsMode { kRowsB = 0, kRowsA = 1 };

// One thread per 8 consecutive features of one token row (rows-B or rows-A).
__global__ __launch_bounds__(256) void pack_rows_kernel(const bf16* __restrict__ src,
                                                        bf16* __restrict__ dst, int mode, int B,
                                                        int N, int Np, int H, int dk) {
  const int d = H * dk, cpr = d / 8;
  const long long s = (long long)blockIdx.x * 256 + threadIdx.x;
  if (s >= (long long)B * Np * cpr) return;
  const long long prow = s / cpr;
  const int col = (int)(s - prow * cpr) * 8;
  const int b = (int)(prow / Np), pos = (int)(prow - (long long)b * Np);
  float v[8];
  if (pos < N) load8_f32(src + ((size_t)b * N + pos) * d + col, v);
  else
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.f;
  size_t frag;
  int slot;
  if (mode == kRowsB) {
    frag = (size_t)(prow >> 5) * (d / 16) + (col >> 4);
    slot = 32 * ((col >> 3) & 1) + (int)(prow & 31);
  } else {
    const int h = col / dk, j = col - h * dk;
    frag = (((size_t)b * H + h) * (Np / 32) + (pos >> 5)) * (dk / 16) + (j >> 4);
    slot = 32 * ((j >> 3) & 1) + pi_row(pos & 31);
  }
  st_packed(dst + frag * kFragElems, slot, v);
}

// The inverse of rows-B for the real rows: packed [B Np, d] -> row-major [B N, d].
__global__ __launch_bounds__(256) void unpack_rows_kernel(const bf16* __restrict__ src,
                                                          bf16* __restrict__ dst, int B, int N,
                                                          int Np, int d) {
  const int cpr = d / 8;
  const long long s = (long long)blockIdx.x * 256 + threadIdx.x;
  if (s >= (long long)B * N * cpr) return;
  const long long row = s / cpr;
  const int col = (int)(s - row * cpr) * 8;
  const int b = (int)(row / N), pos = (int)(row - (long long)b * N);
  const long long prow = (long long)b * Np + pos;
  const size_t frag = (size_t)(prow >> 5) * (d / 16) + (col >> 4);
  const int slot = 32 * ((col >> 3) & 1) + (int)(prow & 31);
  *reinterpret_cast<bf16x8*>(dst + row * d + col) = ld_packed(src + frag * kFragElems, slot);
}

}  // namespace
}  // namespace bpt
