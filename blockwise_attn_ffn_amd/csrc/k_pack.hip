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
// work items [first_item[m], first_item[m+1]) of the grid.
template <typename T>
struct PackJob {
  const T* src[6];
  T* dst[6];
  int rows[6], K[6], order[6];
  long long first_item[7];
  FfnStream fs;
};

// One wave per work item = one 32-row tile and kPackSteps consecutive k-steps:
// lane 32 hf + rho reads W[32 tile + pi(rho)][16 ks + 8 hf .. + 8] for each k-step
// (a row's reads over the item are 256 contiguous bytes) and each k-step's
// fragment is written as 1 KB of contiguous memory.
constexpr int kPackSteps = 8;

template <typename T>
__global__ __launch_bounds__(256) void pack_frag_kernel(PackJob<T> job) {
  const long long item = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= job.first_item[6]) return;
  const int lane = threadIdx.x & 63, hf = lane >> 5, rho = lane & 31;
  int m = 0;
#pragma unroll
  for (int q = 1; q < 6; ++q) m += item >= job.first_item[q];
  const long long li = item - job.first_item[m];
  const int K = job.K[m], ksteps = K / 16;
  const int groups = ksteps / kPackSteps;               // items per row tile
  const int tile = (int)(li / groups), ks0 = (int)(li - (long long)tile * groups) * kPackSteps;
  const int row = 32 * tile + pi_row(rho);              // pi is its own inverse
  const T* src = job.src[m] + (size_t)row * K + 16 * ks0 + 8 * hf;
  const int order = job.order[m];
#pragma unroll
  for (int j = 0; j < kPackSteps; ++j) {
    const int ks = ks0 + j;
    size_t slot;
    if (order == kStreamWO) slot = job.fs.slot_wo(tile, ks);
    else if (order == kStreamW1) slot = job.fs.slot_w1(tile, ks);
    else if (order == kStreamW2) slot = job.fs.slot_w2(tile, ks);
    else slot = (size_t)tile * ksteps + ks;
    st_packed_chunk(job.dst[m] + slot * kFragElems, lane, ld_chunk(src + 16 * j));
  }
}

// Packed region: W_Q, W_K, W_V (one [d + 2 kvp, d] operand: W_K and W_V hold d_kv =
// n_kv_heads * d_head rows each, at offsets d and d + kvp, kvp = d_kv rounded up to
// a product tile; the rows in between are never written and the product's
// features there are dropped), then the epilogue stream holding W_O, W_1 and W_2 (d^2 + 2 d d_ff
// elements); for the staged epilogue W_O, W_1, W_2 in plain fragment order instead.
template <typename T>
int pack_all(const LayerLaunch& L, hipStream_t s, char* err, size_t n) {
  const int d = L.d_model, f = L.d_ff, dkv = L.d_kv, kvp = L.kv_pad;
  const size_t dd = (size_t)d * d, qkv = qkv_pack_elems(d, kvp);
  T* p = static_cast<T*>(L.wpack);
  PackJob<T> job{};
  job.fs = FfnStream{d, f};
  const void* srcs[6] = {L.w.w_q, L.w.w_k, L.w.w_v, L.w.w_o, L.w.w_1, L.w.w_2};
  const bool staged = plain_epilogue_weights(d, L.split, f);
  T* dsts[6] = {p, p + dd, p + dd + (size_t)kvp * d, p + qkv, p + qkv, p + qkv};
  const int rows[6] = {d, dkv, dkv, d, f, d}, Ks[6] = {d, d, d, d, d, f};
  int orders[6] = {kPlain, kPlain, kPlain, kStreamWO, kStreamW1, kStreamW2};
  if (staged) {   // the cooperative and staged epilogues take W_O, W_1, W_2 in plain order
    dsts[4] = p + qkv + dd;
    dsts[5] = p + qkv + dd + (size_t)f * d;
    orders[3] = orders[4] = orders[5] = kPlain;
  }
  job.first_item[0] = 0;
  for (int m = 0; m < 6; ++m) {
    // rows are multiples of 32 and K of 16 * kPackSteps for every width supported
    if (rows[m] % 32 != 0 || Ks[m] % (16 * kPackSteps) != 0) {
      set_err(err, n, "weight shape not a multiple of the packing item%s", "");
      return 1;
    }
    job.src[m] = static_cast<const T*>(srcs[m]);
    job.dst[m] = dsts[m];
    job.rows[m] = rows[m];
    job.K[m] = Ks[m];
    job.order[m] = orders[m];
    job.first_item[m + 1] = job.first_item[m] + (long long)(rows[m] / 32) * (Ks[m] / (16 * kPackSteps));
  }
  const long long total = job.first_item[6];
  hipLaunchKernelGGL(pack_frag_kernel<T>, dim3((unsigned)((total + 3) / 4)), dim3(256), 0, s, job);
  return check_launch("pack_frag", err, n);
}

int launch_pack(const LayerLaunch& L, hipStream_t s, char* err, size_t n) {
  return L.compute_f32 ? pack_all<float>(L, s, err, n) : pack_all<bf16>(L, s, err, n);
}

}  // namespace bpt
