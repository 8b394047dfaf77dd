// Cooperative fused epilogue of the BPT layer for wide layers (d_model 2048 and
// 4096, bf16 operands): output projection, residual, LN2, FFN W_1 -> GELU -> W_2
// and the second residual, with the FFN hidden state kept on chip.
//
// "Blockwise Parallel Transformer — BPT" (aicassindra.com): section "The fused
// blockwise algorithm" (a query block's attention output is finished by W_O and
// the residual, LN and the FFN, and its hidden state is dropped once the
// block's output rows exist), "FLOPs are unchanged — so where is the win?" (the
// hidden state is produced and consumed in fast memory instead of making a trip
// through DRAM) and "Choosing the block size: arithmetic intensity" (each weight
// byte read serves as many FLOPs as the block has rows).
//
// Why cooperative: one compute unit cannot hold a row tile's fp32 accumulator
// [rows, d] once d reaches 2048 (the register file is 512 KB), and fewer rows per
// tile means fewer FLOPs per weight byte than L2 can feed. So G = d / 512
// workgroups, one per compute unit of one XCD (whose L2 they share), form a
// cluster that finishes a tile of 128 rows together. Member g keeps the
// accumulator of output features [512 g, 512 (g + 1)) for all 128 rows in
// registers, from Y through Z, and reads only its slice of W_O and W_2: every
// weight byte it streams serves 128 rows. The members exchange, through a small
// per-cluster region that lives in their XCD's L2:
//   * per-row LN2 partial statistics (mean and squared deviations of the slice),
//     combined exactly into the row's mean and variance;
//   * LN2(Y) of the slice, the W_1 product's operand, which needs all d features;
//   * the hidden chunk: the d_ff axis runs in chunks of 256 G units; member g
//     computes units [256 g, 256 (g + 1)) of a chunk (W_1 over all d), applies
//     GELU and posts them; the W_2 product of the chunk then reads all 256 G
//     units. A chunk lives in the region until the next-but-one chunk replaces
//     it: the [rows, d_ff] hidden state never exists, only [128, 256 G] slices.
// Each exchange is: plain stores, a wait for their completion, one counter
// increment per member (agent-scope atomic); the readers wait (bounded) for G
// increments and read through the L2 with loads that bypass the L1. The members
// of a cluster are found at run time by XCD id, so the exchange never leaves an
// L2. Every wait is bounded: on a timeout the workgroup stops waiting, records
// the failure in the counters' error word and writes NaN for its Z rows.
//
// Products: C^T = W A^T on packed matrix-core fragments (bpt_device.hpp), 8
// waves, operands copied global -> LDS by the LDS-DMA path into three 40 KB
// stages (two k-blocks in flight while one is multiplied).
#include <type_traits>

#include "bpt_device.hpp"
#include "bpt_launch.hpp"

namespace bpt {

struct CoopArgs {
  const void* x;          // residual X [batch * N, d] (real rows), TX
  const bf16* o;          // attention output: packed B fragments [packed rows / 32][d / 16]
  const bf16* o_lo;       // its lo half (bf16 pairs), same layout
  const bf16* w_o;        // plain fragment order [d / 32 tiles][d / 16 k-steps]
  const bf16* w_1;        // [d_ff / 32][d / 16]
  const bf16* w_2;        // [d / 32][d_ff / 16]
  const bf16* ln_g;       // LN2 gain and bias [d]
  const bf16* ln_b;
  void* z;                // Z [batch * N, d] (real rows), TO
  unsigned char* xbuf;    // exchange regions, kCoopRegionBytes(d) per cluster
  unsigned* ctr;          // counters, zero at launch
  int N, Np, n_tiles, d_ff, per_xcc, n_xcc;
  unsigned spin_limit;
  float eps;
};

namespace {

constexpr int kRows = kCoopRows;           // 128 rows per tile
constexpr int kRT = kRows / 32;            // 4 row tiles of 32
constexpr int kNW = 8;                     // waves
// bytes per LDS stage: NA activation halves (8 KB each) and 32 KB of weights
template <bool SPLIT>
constexpr int stage_bytes() { return (SPLIT ? 16 : 8) * 1024 + 32 * 1024; }

// The XCD (XCC) this wave runs on (hardware register XCC_ID, bits 3:0).
__device__ inline unsigned xcc_id() {
  return __builtin_amdgcn_s_getreg((20) | (0 << 6) | ((16 - 1) << 11)) & 0xfu;
}

// 16 bytes per lane into LDS, served by the L2 (the load bypasses the L1, whose
// copy of another compute unit's exchange data could be stale).
__device__ inline void dma16_l2(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)dst, 16, 0, 1);
}

// Wait until at most N of this wave's vector-memory operations (its LDS copies)
// are outstanding and its LDS reads have returned.
template <int N>
__device__ inline void wait_vmem_upto() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0070 | N);
}

// Workgroup barrier without a memory fence. __syncthreads() also releases this
// wave's memory operations, which makes every wave wait for all of its LDS copies
// in flight (the copies of the k-blocks ahead) before the barrier. Here each wave
// has waited for exactly the copies that must have landed; the empty asm
// statements keep the compiler from moving memory accesses across the barrier.
__device__ inline void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS byte address of a pointer into a __shared__ array (the low half of its
// flat address).
__device__ inline uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

// Fragment reads of one k-block from a stage, written as assembly with the wait
// for their data in the same statement. Reads expressed in C++ after copies into
// LDS are in flight make the compiler wait for every copy (it cannot tell that the
// three stages do not overlap once a loop carries the copies around), which would
// serialise the pipeline; these reads are ordered by the stage barriers instead.
// 12 fragments: a[j][b] at abase + (4 j + b) KB, w[j][t] at wbase + (2 t + j) KB.
__device__ inline void ld_stage12(uint32_t abase, uint32_t wbase, bf16x8 (&a)[2][4], bf16x8 (&w)[2][2]) {
  asm volatile(
      "ds_read_b128 %0, %12 offset:0\n\t"
      "ds_read_b128 %1, %12 offset:1024\n\t"
      "ds_read_b128 %2, %12 offset:2048\n\t"
      "ds_read_b128 %3, %12 offset:3072\n\t"
      "ds_read_b128 %4, %12 offset:4096\n\t"
      "ds_read_b128 %5, %12 offset:5120\n\t"
      "ds_read_b128 %6, %12 offset:6144\n\t"
      "ds_read_b128 %7, %12 offset:7168\n\t"
      "ds_read_b128 %8, %13 offset:0\n\t"
      "ds_read_b128 %9, %13 offset:2048\n\t"
      "ds_read_b128 %10, %13 offset:1024\n\t"
      "ds_read_b128 %11, %13 offset:3072\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=v"(a[0][0]), "=v"(a[0][1]), "=v"(a[0][2]), "=v"(a[0][3]), "=v"(a[1][0]), "=v"(a[1][1]),
        "=v"(a[1][2]), "=v"(a[1][3]), "=v"(w[0][0]), "=v"(w[0][1]), "=v"(w[1][0]), "=v"(w[1][1])
      : "v"(abase), "v"(wbase));
}
// 8 fragments: a[j][b] at abase + (4 j + b) KB (b < 2), w[j][t] at wbase + (2 t + j) KB.
__device__ inline void ld_stage8(uint32_t abase, uint32_t wbase, bf16x8 (&a)[2][2], bf16x8 (&w)[2][2]) {
  asm volatile(
      "ds_read_b128 %0, %8 offset:0\n\t"
      "ds_read_b128 %1, %8 offset:1024\n\t"
      "ds_read_b128 %2, %8 offset:4096\n\t"
      "ds_read_b128 %3, %8 offset:5120\n\t"
      "ds_read_b128 %4, %9 offset:0\n\t"
      "ds_read_b128 %5, %9 offset:2048\n\t"
      "ds_read_b128 %6, %9 offset:1024\n\t"
      "ds_read_b128 %7, %9 offset:3072\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=v"(a[0][0]), "=v"(a[0][1]), "=v"(a[1][0]), "=v"(a[1][1]), "=v"(w[0][0]), "=v"(w[0][1]),
        "=v"(w[1][0]), "=v"(w[1][1])
      : "v"(abase), "v"(wbase));
}

// One k-step of the pair mode: act hi [4] at abase + b KB, act lo [4] at abase +
// 8 KB + b KB, weights [2] at wbase + 2 t KB.
__device__ inline void ld_step10(uint32_t abase, uint32_t wbase, bf16x8 (&a)[4], bf16x8 (&al)[4],
                                 bf16x8 (&w)[2]) {
  asm volatile(
      "ds_read_b128 %0, %10 offset:0\n\t"
      "ds_read_b128 %1, %10 offset:1024\n\t"
      "ds_read_b128 %2, %10 offset:2048\n\t"
      "ds_read_b128 %3, %10 offset:3072\n\t"
      "ds_read_b128 %4, %10 offset:8192\n\t"
      "ds_read_b128 %5, %10 offset:9216\n\t"
      "ds_read_b128 %6, %10 offset:10240\n\t"
      "ds_read_b128 %7, %10 offset:11264\n\t"
      "ds_read_b128 %8, %11 offset:0\n\t"
      "ds_read_b128 %9, %11 offset:2048\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=v"(a[0]), "=v"(a[1]), "=v"(a[2]), "=v"(a[3]), "=v"(al[0]), "=v"(al[1]), "=v"(al[2]),
        "=v"(al[3]), "=v"(w[0]), "=v"(w[1])
      : "v"(abase), "v"(wbase));
}
// act hi [2] at abase + b KB, act lo [2] at abase + 8 KB + b KB, weights [2] at wbase + 2 t KB.
__device__ inline void ld_step6(uint32_t abase, uint32_t wbase, bf16x8 (&a)[2], bf16x8 (&al)[2],
                                bf16x8 (&w)[2]) {
  asm volatile(
      "ds_read_b128 %0, %6 offset:0\n\t"
      "ds_read_b128 %1, %6 offset:1024\n\t"
      "ds_read_b128 %2, %6 offset:8192\n\t"
      "ds_read_b128 %3, %6 offset:9216\n\t"
      "ds_read_b128 %4, %7 offset:0\n\t"
      "ds_read_b128 %5, %7 offset:2048\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=v"(a[0]), "=v"(a[1]), "=v"(al[0]), "=v"(al[1]), "=v"(w[0]), "=v"(w[1])
      : "v"(abase), "v"(wbase));
}

// v as a bf16 pair: hi = v rounded to bf16 at p, lo = v - hi rounded at plo.
__device__ inline void st_pair_packed(bf16* p, bf16* plo, int lane, float* v, bool split) {
  st_packed(p, lane, v);
  if (split) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] -= bf16_round(v[e]);
    st_packed(plo, lane, v);
  }
}

__device__ inline void post(unsigned* c) {
  __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Bounded wait of one thread until *c >= want. False on a timeout, or when some
// workgroup has already recorded a failure (then nobody waits any more).
__device__ inline bool wait_count(unsigned* c, unsigned want, unsigned* err, unsigned limit) {
  for (unsigned i = 0;; ++i) {
    if (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= want) return true;
    if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u || i >= limit) {
      __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

__device__ inline float2 load_l2_f2(const float2* p) {
  const unsigned long long u = __hip_atomic_load(reinterpret_cast<const unsigned long long*>(p),
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((unsigned)u), __uint_as_float((unsigned)(u >> 32)));
}

}  // namespace

template <typename TX, typename TO, int G, bool SPLIT>
__global__ __launch_bounds__(512, 1) void ffn_coop_kernel(CoopArgs a) {
  using O = Op<bf16>;
  using F = O::frag;
  constexpr int D = kCoopCols * G;         // d_model
  constexpr int HC = kCoopUnits * G;       // hidden units per chunk
  constexpr int KSD = D / 16, KSH = HC / 16;
  constexpr int NKB_D = D / 32, NKB_H = HC / 32;   // k-blocks of 2 k-steps
  constexpr int OWN_D = kCoopCols / 32;    // k-blocks of d that are this member's features
  constexpr int OWN_H = kCoopUnits / 32;   // k-blocks of a chunk that are this member's units
  constexpr int NA = SPLIT ? 2 : 1;        // activation halves: hi, and lo for bf16 pairs
  constexpr int AKB = 8 * NA;              // KB of activation fragments per stage
  constexpr int CPZ = NA + 4, CPU = NA + 2;   // copies per wave per stage (Z side, W_1)
  constexpr int kStage = stage_bytes<SPLIT>();
  constexpr CoopRegion R{D, HC, G, NA};
  // three distinct stage arrays (not one indexed array): the compiler then sees
  // that copies into one stage never alias reads of another, and does not wait for
  // the copies in flight before reading the current stage
  __shared__ __align__(16) unsigned char st0[kStage];
  __shared__ __align__(16) unsigned char st1[kStage];
  __shared__ __align__(16) unsigned char st2[kStage];
  __shared__ float red[kNW][kRows];
  __shared__ float2 rowstat[kRows];
  __shared__ int s_cluster, s_member, s_failed;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rho = lane & 31, hf = lane >> 5;
  unsigned* const err = a.ctr + kCoopCtrError;

  if (tid == 0) {
    const unsigned x = xcc_id() % (unsigned)a.n_xcc;
    const unsigned t = __hip_atomic_fetch_add(&a.ctr[kCoopCtrTickets + x], 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    if (t < (unsigned)a.per_xcc) {
      s_cluster = (int)(x * (unsigned)(a.per_xcc / G) + t / G);
      s_member = (int)(t % G);
      s_failed = 0;
    } else {   // more workgroups on this XCD than planned: no cluster to join
      __hip_atomic_fetch_or(err, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_cluster = -1;
      s_member = 0;
      s_failed = 1;
    }
  }
  __syncthreads();
  const int cluster = s_cluster, g = s_member;
  if (cluster < 0) return;
  const int n_clusters = a.n_xcc * (a.per_xcc / G);
  unsigned char* const region = a.xbuf + (size_t)cluster * R.bytes();
  bf16* const A = reinterpret_cast<bf16*>(region + R.a_off());      // [NA][kRT][KSD] fragments
  bf16* const H = reinterpret_cast<bf16*>(region + R.h_off());      // [2][NA][kRT][KSH] fragments
  constexpr size_t A_HALF = (size_t)kRT * KSD * kFragElems, H_HALF = (size_t)kRT * KSH * kFragElems;
  float2* const S = reinterpret_cast<float2*>(region + R.s_off());  // [2][G][kRows]
  unsigned* const c_stats = a.ctr + kCoopCtrCluster + 4 * cluster;
  unsigned* const c_a = c_stats + 1;
  unsigned* const c_h = c_stats + 2;
  const int n_chunks = a.d_ff / HC;
  const int KS2 = a.d_ff / 16;

  // Z-side wave tiles: feature tiles zt0, zt0 + 1 of the member's 16, all row tiles.
  const int zt0 = 2 * wave;
  // hidden-side wave tiles: unit tiles ut0, ut0 + 1 of the member's 8, row tiles rb0, rb0 + 1.
  const int ut0 = 2 * (wave & 3), rb0 = 2 * (wave >> 2);

  f32x16 acc[2][kRT];    // [feature tile][row tile]: Y, then Z, of the member's slice
  bool failed = false;

  // A pipelined product phase over n_kb k-blocks: copy(kb, stage) issues this
  // wave's CP LDS copies of k-block kb, compute(stage) multiplies one k-block,
  // hook(kb) runs before the barrier of iteration kb (exchange waits).
  auto phase = [&](int n_kb, auto cp_c, auto copy, auto compute, auto hook)
      __attribute__((always_inline)) {
    constexpr int CP = decltype(cp_c)::value;
    // k-block kb is multiplied from stage kb % 3 while kb + 1 and kb + 2 are in flight
    auto step = [&](int kb, unsigned char* cur, unsigned char* ahead2) __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);   // the previous k-block's products stay before the wait
      if (kb + 1 < n_kb) wait_vmem_upto<CP>();
      else wait_vmem_upto<0>();
      hook(kb);
      stage_barrier();   // k-block kb landed for every wave; stage (kb + 2) % 3 is free
      // the copies of k-block kb + 2 are issued once the first k-step's fragments
      // have been read (their address registers are then not needed by the reads)
      compute(cur, [&]() __attribute__((always_inline)) {
        if (kb + 2 < n_kb) copy(kb + 2, ahead2);
      });
    };
    copy(0, st0);
    copy(1, st1);
    int kb = 0;
    for (; kb + 3 <= n_kb; kb += 3) {
      step(kb, st0, st2);
      step(kb + 1, st1, st0);
      step(kb + 2, st2, st1);
    }
    if (kb < n_kb) step(kb, st0, st2);
    if (kb + 1 < n_kb) step(kb + 1, st1, st0);
    __syncthreads();     // stages free for the next phase
  };
  // The copies of one k-block: activation fragments (half hh, row tile b, k-step
  // j) at stage byte (8 hh + 4 j + b) KB, weight fragments (tile t, k-step j) at
  // (AKB + 2 t + j) KB; copy idx of a k-block lands at idx KB.
  auto zcompute = [&](const unsigned char* st, auto issue) __attribute__((always_inline)) {
    if constexpr (!SPLIT) {
      F af[2][kRT], wf[2][2];
      ld_stage12(lds_addr(st) + lane * 16, lds_addr(st) + AKB * 1024 + zt0 * 2048 + lane * 16, af, wf);
      __builtin_amdgcn_sched_barrier(0);
      issue();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int b = 0; b < kRT; ++b) O::mma(acc[t][b], wf[j][t], af[j][b]);
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        F af[kRT], al[kRT], wf[2];
        ld_step10(lds_addr(st) + j * 4096 + lane * 16, lds_addr(st) + AKB * 1024 + zt0 * 2048 + j * 1024 + lane * 16,
                  af, al, wf);
        if (j == 0) {
          __builtin_amdgcn_sched_barrier(0);
          issue();
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int b = 0; b < kRT; ++b) {
            O::mma(acc[t][b], wf[t], af[b]);
            O::mma(acc[t][b], wf[t], al[b]);
          }
      }
    }
  };
  auto no_hook = [](int) {};

  for (int it = 0, tile = cluster; tile < a.n_tiles; ++it, tile += n_clusters) {
    const int r0 = tile * kRows;
    const int seq = r0 / a.Np, pos0 = r0 - seq * a.Np;

    // ---- accumulators start at the residual X (padding rows read a real row)
#pragma unroll
    for (int b = 0; b < kRT; ++b) {
      const int pos = min(pos0 + b * 32 + rho, a.N - 1);
      const TX* xr = static_cast<const TX*>(a.x) + ((size_t)seq * a.N + pos) * D + g * kCoopCols;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
          float xv[8];
          load8_f32(xr + (zt0 + t) * 32 + 16 * gg + 8 * hf, xv);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[t][b][8 * gg + e] = xv[e];
        }
    }

    // ---- Y^T = X^T + W_O[slice] O^T over all d
    {
      const bf16* osrc = a.o + (size_t)(r0 / 32) * KSD * kFragElems;
      const bf16* osrc_lo = SPLIT ? a.o_lo + (size_t)(r0 / 32) * KSD * kFragElems : osrc;
      const bf16* wsrc = a.w_o + (size_t)(g * 16) * KSD * kFragElems;
      // copy q of this wave: fragment (row tile or weight tile, k-step j) of
      // k-block 0; k-block kb is 2 kb fragments further
      const char* base[CPZ];
#pragma unroll
      for (int q = 0; q < CPZ; ++q) {
        const int idx = wave * CPZ + q, i = idx & 7;
        base[q] = reinterpret_cast<const char*>(
            idx < AKB ? (idx < 8 ? osrc : osrc_lo) + ((size_t)(i & 3) * KSD + (i >> 2)) * kFragElems
                      : wsrc + ((size_t)((idx - AKB) >> 1) * KSD + ((idx - AKB) & 1)) * kFragElems);
      }
      auto copy = [&](int kb, unsigned char* st) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < CPZ; ++q)
          dma16_l2(base[q] + (size_t)kb * 2048 + lane * 16, st + (wave * CPZ + q) * 1024);
      };
      phase(NKB_D, std::integral_constant<int, CPZ>{}, copy, zcompute, no_hook);
    }

    // ---- LN2 statistics of every row: this member's slice, then the cluster's
    const int par = it & 1;
#pragma unroll
    for (int b = 0; b < kRT; ++b) {
      float s = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) s += acc[t][b][i];
      s += __shfl_xor(s, 32, 64);
      if (hf == 0) red[wave][b * 32 + rho] = s;
    }
    __syncthreads();
    if (tid < kRows) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < kNW; ++w) s += red[w][tid];
      rowstat[tid].x = s * (1.0f / kCoopCols);     // mean of the slice
    }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < kRT; ++b) {
      const float m = rowstat[b * 32 + rho].x;
      float q = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float dv = acc[t][b][i] - m;
          q += dv * dv;
        }
      q += __shfl_xor(q, 32, 64);
      if (hf == 0) red[wave][b * 32 + rho] = q;
    }
    __syncthreads();
    if (tid < kRows) {
      float q = 0.f;
#pragma unroll
      for (int w = 0; w < kNW; ++w) q += red[w][tid];
      S[((size_t)par * G + g) * kRows + tid] = make_float2(rowstat[tid].x, q);
    }
    wait_vmem();
    __syncthreads();
    if (tid == 0) {
      post(c_stats);
      if (!s_failed && !wait_count(c_stats, (unsigned)G * (it + 1), err, a.spin_limit)) s_failed = 1;
    }
    __syncthreads();
    if (tid < kRows) {
      // exact merge of equal-size slices: mean = avg of means, M2 = sum M2 + n sum (m_g - mean)^2
      float2 p[G];
#pragma unroll
      for (int m = 0; m < G; ++m) p[m] = load_l2_f2(&S[((size_t)par * G + m) * kRows + tid]);
      float mean = 0.f;
#pragma unroll
      for (int m = 0; m < G; ++m) mean += p[m].x;
      mean *= 1.0f / G;
      float m2 = 0.f, dm = 0.f;
#pragma unroll
      for (int m = 0; m < G; ++m) {
        m2 += p[m].y;
        const float e = p[m].x - mean;
        dm += e * e;
      }
      m2 += (float)kCoopCols * dm;
      rowstat[tid] = make_float2(mean, 1.0f / sqrtf(m2 * (1.0f / D) + a.eps));
    }
    __syncthreads();
    failed = failed || s_failed;

    // ---- LN2(Y) of the slice -> the cluster's A fragments
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        const int n = g * kCoopCols + (zt0 + t) * 32 + 16 * gg + 8 * hf;
        float gv[8], bv[8];
        load8_f32(a.ln_g + n, gv);
        load8_f32(a.ln_b + n, bv);
#pragma unroll
        for (int b = 0; b < kRT; ++b) {
          const float2 st = rowstat[b * 32 + rho];
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = (acc[t][b][8 * gg + e] - st.x) * st.y * gv[e] + bv[e];
          const size_t f = ((size_t)b * KSD + (n >> 4)) * kFragElems;
          st_pair_packed(A + f, A + A_HALF + f, lane, v, SPLIT);
        }
      }
    wait_vmem();
    __syncthreads();
    if (tid == 0) post(c_a);

    // ---- FFN over hidden chunks
    for (int c = 0; c < n_chunks; ++c) {
      const int gc = it * n_chunks + c;          // chunks posted so far by every member
      const int hp = gc & 1;
      // U^T = W_1[member's units of chunk c] LN2(Y)^T, k over d starting at the own slice
      f32x16 u[2][2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int b = 0; b < 2; ++b) u[t][b] = f32x16{};
      {
        const bf16* w1src = a.w_1 + (size_t)(c * 8 * G + 8 * g) * KSD * kFragElems;
        const char* base[CPU];
#pragma unroll
        for (int q = 0; q < CPU; ++q) {
          const int idx = wave * CPU + q, i = idx & 7;
          base[q] = reinterpret_cast<const char*>(
              idx < AKB ? A + (idx < 8 ? 0 : A_HALF) + ((size_t)(i & 3) * KSD + (i >> 2)) * kFragElems
                        : w1src + ((size_t)((idx - AKB) >> 1) * KSD + ((idx - AKB) & 1)) * kFragElems);
        }
        auto copy = [&](int kb, unsigned char* st) __attribute__((always_inline)) {
          const int kp = (kb + OWN_D * g) % NKB_D;
#pragma unroll
          for (int q = 0; q < CPU; ++q)
            dma16_l2(base[q] + (size_t)kp * 2048 + lane * 16, st + (wave * CPU + q) * 1024);
        };
        auto compute = [&](const unsigned char* st, auto issue) __attribute__((always_inline)) {
          if constexpr (!SPLIT) {
            F af[2][2], wf[2][2];
            ld_stage8(lds_addr(st) + rb0 * 1024 + lane * 16, lds_addr(st) + AKB * 1024 + ut0 * 2048 + lane * 16,
                      af, wf);
            __builtin_amdgcn_sched_barrier(0);
            issue();
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
              for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int b = 0; b < 2; ++b) O::mma(u[t][b], wf[j][t], af[j][b]);
          } else {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              F af[2], al[2], wf[2];
              ld_step6(lds_addr(st) + j * 4096 + rb0 * 1024 + lane * 16,
                       lds_addr(st) + AKB * 1024 + ut0 * 2048 + j * 1024 + lane * 16, af, al, wf);
              if (j == 0) {
                __builtin_amdgcn_sched_barrier(0);
                issue();
                __builtin_amdgcn_sched_barrier(0);
              }
#pragma unroll
              for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                  O::mma(u[t][b], wf[t], af[b]);
                  O::mma(u[t][b], wf[t], al[b]);
                }
            }
          }
        };
        // the other members' features of LN2(Y) are needed from k-block OWN_D on
        auto hook = [&](int kb) __attribute__((always_inline)) {
          if (c == 0 && kb + 2 == OWN_D && tid == 0 && !s_failed &&
              !wait_count(c_a, (unsigned)G * (it + 1), err, a.spin_limit))
            s_failed = 1;
        };
        phase(NKB_D, std::integral_constant<int, CPU>{}, copy, compute, hook);
      }
      // H = GELU(U) -> the member's units of the chunk in the cluster's hidden buffer
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
          const int ks = 16 * g + 2 * (ut0 + t) + gg;   // k-step of the chunk
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = gelu_tanh(u[t][b][8 * gg + e]);
            const size_t f = (size_t)hp * NA * H_HALF + ((size_t)(rb0 + b) * KSH + ks) * kFragElems;
            st_pair_packed(H + f, H + H_HALF + f, lane, v, SPLIT);
          }
        }
      wait_vmem();
      __syncthreads();
      if (tid == 0) post(c_h);
      // Z^T += W_2[slice, chunk] H^T, k over the chunk starting at the own units
      {
        const bf16* hsrc = H + (size_t)hp * NA * H_HALF;
        const bf16* w2src = a.w_2 + ((size_t)(g * 16) * KS2 + (size_t)c * KSH) * kFragElems;
        const char* base[CPZ];
#pragma unroll
        for (int q = 0; q < CPZ; ++q) {
          const int idx = wave * CPZ + q, i = idx & 7;
          base[q] = reinterpret_cast<const char*>(
              idx < AKB ? hsrc + (idx < 8 ? 0 : H_HALF) + ((size_t)(i & 3) * KSH + (i >> 2)) * kFragElems
                        : w2src + ((size_t)((idx - AKB) >> 1) * KS2 + ((idx - AKB) & 1)) * kFragElems);
        }
        auto copy = [&](int kb, unsigned char* st) __attribute__((always_inline)) {
          const int kp = (kb + OWN_H * g) % NKB_H;
#pragma unroll
          for (int q = 0; q < CPZ; ++q)
            dma16_l2(base[q] + (size_t)kp * 2048 + lane * 16, st + (wave * CPZ + q) * 1024);
        };
        // the other members' units of the chunk are needed from k-block OWN_H on
        auto hook = [&](int kb) __attribute__((always_inline)) {
          if (kb + 2 == OWN_H && tid == 0 && !s_failed &&
              !wait_count(c_h, (unsigned)G * (gc + 1), err, a.spin_limit))
            s_failed = 1;
        };
        phase(NKB_H, std::integral_constant<int, CPZ>{}, copy, zcompute, hook);
      }
    }
    failed = failed || s_failed;

    // ---- Z = Y + H W_2 for the slice (real rows only; NaN after a failed wait)
#pragma unroll
    for (int b = 0; b < kRT; ++b) {
      const int pos = pos0 + b * 32 + rho;
      if (pos >= a.N) continue;
      TO* zr = static_cast<TO*>(a.z) + ((size_t)seq * a.N + pos) * D + g * kCoopCols;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = failed ? __builtin_nanf("") : acc[t][b][8 * gg + e];
          store8_f32(zr + (zt0 + t) * 32 + 16 * gg + 8 * hf, v);
        }
    }
  }
}

namespace {

__global__ void zero_words_kernel(unsigned* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

template <typename TX, typename TO, int G, bool SPLIT>
int run_coop(const LayerLaunch& L, hipStream_t s, char* err, size_t n) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
    set_err(err, n, "cooperative epilogue: no device attributes%s", "");
    return 1;
  }
  // workgroups are dispatched round-robin over the XCDs: per_xcc of them per XCD,
  // a multiple of the cluster size, at most the compute units of an XCD
  const int n_xcc = kCoopXcds;
  int per_xcc = (cus / n_xcc) / G * G;
  if (per_xcc * n_xcc > kCoopMaxWorkgroups) per_xcc = kCoopMaxWorkgroups / n_xcc / G * G;
  if (per_xcc < G) {
    set_err(err, n, "cooperative epilogue: too few compute units (%s%d)", "", cus);
    return 1;
  }
  hipLaunchKernelGGL(zero_words_kernel, dim3(1), dim3(256), 0, s, static_cast<unsigned*>(L.coop_ctr),
                     kCoopCtrWords);
  if (check_launch("coop_zero", err, n)) return 1;
  CoopArgs a{};
  const int d = L.d_model;
  const size_t dd = (size_t)d * d, qkv = qkv_pack_elems(d, L.kv_pad);
  const bf16* wp = static_cast<const bf16*>(L.wpack);
  a.x = L.x;
  a.o = static_cast<const bf16*>(L.q);
  a.o_lo = static_cast<const bf16*>(L.q_lo);
  a.w_o = wp + qkv;
  a.w_1 = wp + qkv + dd;
  a.w_2 = wp + qkv + dd + (size_t)L.d_ff * d;
  a.ln_g = static_cast<const bf16*>(L.w.ln2_g);
  a.ln_b = static_cast<const bf16*>(L.w.ln2_b);
  a.z = L.z;
  a.xbuf = static_cast<unsigned char*>(L.coop_buf);
  a.ctr = static_cast<unsigned*>(L.coop_ctr);
  a.N = L.seq_len;
  a.Np = L.seq_pad;
  a.n_tiles = L.batch * L.seq_pad / kCoopRows;
  a.d_ff = L.d_ff;
  a.per_xcc = per_xcc;
  a.n_xcc = n_xcc;
  a.spin_limit = 1u << 22;
  a.eps = L.ln_eps;
  auto k = ffn_coop_kernel<TX, TO, G, SPLIT>;
  void* args[] = {&a};
  hipError_t e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(k), dim3(n_xcc * per_xcc),
                                            dim3(512), args, 0, s);
  if (e != hipSuccess) {
    set_err(err, n, "ffn_coop launch: %s", hipGetErrorString(e));
    return 1;
  }
  return check_launch("ffn_coop", err, n);
}

template <typename TX, typename TO>
int dispatch_coop(const LayerLaunch& L, hipStream_t s, char* err, size_t n) {
  switch (L.d_model) {
    case 2048:
      return L.split ? run_coop<TX, TO, 4, true>(L, s, err, n) : run_coop<TX, TO, 4, false>(L, s, err, n);
    case 4096:
      return L.split ? run_coop<TX, TO, 8, true>(L, s, err, n) : run_coop<TX, TO, 8, false>(L, s, err, n);
    default: break;
  }
  set_err(err, n, "no cooperative epilogue for d_model %s%d", "", L.d_model);
  return 1;
}

}  // namespace

int launch_ffn_coop(const LayerLaunch& L, hipStream_t s, char* err, size_t n) {
  if (L.x_f32)
    return L.z_f32 ? dispatch_coop<float, float>(L, s, err, n) : dispatch_coop<float, bf16>(L, s, err, n);
  return L.z_f32 ? dispatch_coop<bf16, float>(L, s, err, n) : dispatch_coop<bf16, bf16>(L, s, err, n);
}

}  // namespace bpt
