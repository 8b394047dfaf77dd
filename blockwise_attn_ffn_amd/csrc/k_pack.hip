// Repacking of the epilogue's weight matrices into matrix-core fragment order.
//
// A weight W[n][k] (k contiguous, the library's [out, in] layout) is consumed as
// the A operand of 32x32 matrix-core tiles: lane l = 32 * hf + rho holds row
// pi(rho) of a 32-row tile and 8 consecutive k of a 16-wide k-step. Read straight
// from W, one 64-lane load touches 32 rows, i.e. 32 cache lines per instruction,
// and the vector-memory path is bound by lines, not bytes. The packed copy puts
// each (row tile, k-step) fragment in 64 consecutive 8-element chunks in lane
// order (bpt_device.hpp: packed fragments), so one load instruction reads
// contiguous memory:
//
//   fragment (tile, ks) = packed + (tile * (K / 16) + ks) * 512, and in it lane
//   32 * hf + rho holds W[32 * tile + pi(rho)][16 * ks + 8 * hf + e], e = 0..7.
//
// W_O, W_1 and W_2 are not stored matrix by matrix but as the epilogue's
// per-wave weight stream (ffn_stream.hpp): the same fragments, in the order in
// which each epilogue wave consumes them.
#include "bpt_device.hpp"
#include "bpt_launch.hpp"
#include "ffn_stream.hpp"

namespace bpt {

enum PackOrder { kPlain = 0, kStreamWO = 1, kStreamW1 = 2, kStreamW2 = 3 };

// The six matrices of a layer, repacked by one launch: matrix m covers the
// 8-element chunks [first_chunk[m], first_chunk[m+1]) of the grid.
template <typename T>
struct PackJob {
  const T* src[6];
  T* dst[6];
  int rows[6], K[6], order[6];
  long long first_chunk[7];
  FfnStream fs;
};

// One thread per 8-element chunk of a weight; reads are row-contiguous.
template <typename T>
__global__ __launch_bounds__(256) void pack_frag_kernel(PackJob<T> job) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= job.first_chunk[6]) return;
  int m = 0;
#pragma unroll
  for (int q = 1; q < 6; ++q) m += i >= job.first_chunk[q];
  const long long li = i - job.first_chunk[m];
  const int K = job.K[m], kc = K / 8;                     // chunks per row
  const int row = (int)(li / kc), c = (int)(li - (long long)row * kc);
  const int tile = row >> 5, rho = pi_row(row & 31);      // pi is its own inverse
  const int ks = c >> 1, hf = c & 1;
  size_t slot;
  const int order = job.order[m];
  if (order == kStreamWO) slot = job.fs.slot_wo(tile, ks);
  else if (order == kStreamW1) slot = job.fs.slot_w1(tile, ks);
  else if (order == kStreamW2) slot = job.fs.slot_w2(tile, ks);
  else slot = (size_t)tile * (K / 16) + ks;
  st_packed_chunk(job.dst[m] + slot * kFragElems, 32 * hf + rho,
                  ld_chunk(job.src[m] + (size_t)row * K + (size_t)c * 8));
}

// Packed region: W_Q, W_K, W_V (one [3d, d] operand), then the epilogue stream
// holding W_O, W_1 and W_2 (d^2 + 2 d d_ff elements); for the staged epilogue
// W_O, W_1, W_2 in plain fragment order instead.
template <typename T>
int pack_all(const LayerLaunch& L, hipStream_t s, char* err, size_t n) {
  const int d = L.d_model, f = L.d_ff;
  const size_t dd = (size_t)d * d;
  T* p = static_cast<T*>(L.wpack);
  PackJob<T> job{};
  job.fs = FfnStream{d, f};
  const void* srcs[6] = {L.w.w_q, L.w.w_k, L.w.w_v, L.w.w_o, L.w.w_1, L.w.w_2};
  const bool staged = staged_epilogue(d, L.split);
  T* dsts[6] = {p, p + dd, p + 2 * dd, p + 3 * dd, p + 3 * dd, p + 3 * dd};
  const int rows[6] = {d, d, d, d, f, d}, Ks[6] = {d, d, d, d, d, f};
  int orders[6] = {kPlain, kPlain, kPlain, kStreamWO, kStreamW1, kStreamW2};
  if (staged) {   // the staged epilogue's GEMMs take W_O, W_1, W_2 in plain order
    dsts[4] = p + 4 * dd;
    dsts[5] = p + 4 * dd + (size_t)f * d;
    orders[3] = orders[4] = orders[5] = kPlain;
  }
  job.first_chunk[0] = 0;
  for (int m = 0; m < 6; ++m) {
    job.src[m] = static_cast<const T*>(srcs[m]);
    job.dst[m] = dsts[m];
    job.rows[m] = rows[m];
    job.K[m] = Ks[m];
    job.order[m] = orders[m];
    job.first_chunk[m + 1] = job.first_chunk[m] + (long long)rows[m] * (Ks[m] / 8);
  }
  const long long total = job.first_chunk[6];
  hipLaunchKernelGGL(pack_frag_kernel<T>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, job);
  return check_launch("pack_frag", err, n);
}

int launch_pack(const LayerLaunch& L, hipStream_t s, char* err, size_t n) {
  return L.compute_f32 ? pack_all<float>(L, s, err, n) : pack_all<bf16>(L, s, err, n);
}

}  // namespace bpt
