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

// One thread per 8-element chunk of W; reads are row-contiguous.
template <typename T>
__global__ __launch_bounds__(256) void pack_frag_kernel(const T* __restrict__ W, T* __restrict__ P,
                                                        int n_rows, int K, int order, FfnStream fs) {
  const int kc = K / 8;                                   // chunks per row
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)n_rows * kc) return;
  const int row = (int)(i / kc), c = (int)(i - (size_t)row * kc);
  const int tile = row >> 5, rho = pi_row(row & 31);      // pi is its own inverse
  const int ks = c >> 1, hf = c & 1;
  size_t slot;
  if (order == kStreamWO) slot = fs.slot_wo(tile, ks);
  else if (order == kStreamW1) slot = fs.slot_w1(tile, ks);
  else if (order == kStreamW2) slot = fs.slot_w2(tile, ks);
  else slot = (size_t)tile * (K / 16) + ks;
  st_packed_chunk(P + slot * kFragElems, 32 * hf + rho, ld_chunk(W + (size_t)row * K + (size_t)c * 8));
}

namespace {
template <typename T>
int run_pack(const void* W, void* P, int n_rows, int K, int order, FfnStream fs, hipStream_t s,
             char* err, size_t n) {
  const size_t chunks = (size_t)n_rows * (K / 8);
  hipLaunchKernelGGL(pack_frag_kernel<T>, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, s,
                     (const T*)W, (T*)P, n_rows, K, order, fs);
  return check_launch("pack_frag", err, n);
}
}  // namespace

// Packed region: W_Q, W_K, W_V (one [3d, d] operand), then the epilogue stream
// holding W_O, W_1 and W_2 (d^2 + 2 d d_ff elements).
template <typename T>
int pack_all(const LayerLaunch& L, hipStream_t s, char* err, size_t n) {
  const int d = L.d_model, f = L.d_ff;
  const size_t dd = (size_t)d * d;
  const FfnStream fs{d, f};
  T* p = static_cast<T*>(L.wpack);
  return run_pack<T>(L.w.w_q, p, d, d, kPlain, fs, s, err, n) ||
         run_pack<T>(L.w.w_k, p + dd, d, d, kPlain, fs, s, err, n) ||
         run_pack<T>(L.w.w_v, p + 2 * dd, d, d, kPlain, fs, s, err, n) ||
         run_pack<T>(L.w.w_o, p + 3 * dd, d, d, kStreamWO, fs, s, err, n) ||
         run_pack<T>(L.w.w_1, p + 3 * dd, f, d, kStreamW1, fs, s, err, n) ||
         run_pack<T>(L.w.w_2, p + 3 * dd, d, f, kStreamW2, fs, s, err, n);
}

int launch_pack(const LayerLaunch& L, hipStream_t s, char* err, size_t n) {
  return L.compute_f32 ? pack_all<float>(L, s, err, n) : pack_all<bf16>(L, s, err, n);
}

}  // namespace bpt
