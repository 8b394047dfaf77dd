// Attention backward: host launch sequence (the kernels: attn_bwd_kernels.hpp).
// Compiled with the matrix-core results kept in VGPRs (they feed the softmax
// arithmetic at once; the d_k 64 instances are 45% slower without it); the d_k 128
// dK / dV kernel (split by gradient over two waves per SIMD) is instantiated in
// k_attention_bwd_dkv.hip without that setting.
#include "attn_bwd_kernels.hpp"

namespace bpt {

int launch_bwd_dkv128(const BwdArgs& g, int grid, bool general, hipStream_t s);

namespace {

int mark(const AttnBwdLaunch& L, int i, hipStream_t s, char* err, size_t n) {
  if (!L.events) return 0;
  const hipError_t e = hipEventRecord(reinterpret_cast<hipEvent_t>(L.events[i]), s);
  if (e != hipSuccess) {
    set_err(err, n, "hipEventRecord: %s", hipGetErrorString(e));
    return 1;
  }
  return 0;
}

template <int DK>
int run_bwd(const AttnBwdLaunch& L, hipStream_t s, char* err, size_t n) {
  // the kernels' shape assumptions
  if (L.d_model != L.n_heads * DK || L.seq_pad % 128 != 0 || L.seq_pad < L.seq_len || L.seq_len < 1) {
    set_err(err, n, "attention backward: inconsistent launch shape%s (seq_pad %d)", "", L.seq_pad);
    return 1;
  }
  BwdArgs g{};
  g.q = static_cast<const bf16*>(L.q);
  g.k = static_cast<const bf16*>(L.k);
  g.v = static_cast<const bf16*>(L.v);
  g.dout = static_cast<const bf16*>(L.dout);
  bf16* kT = static_cast<bf16*>(L.packed[0]);
  bf16* qT = static_cast<bf16*>(L.packed[1]);
  bf16* doT = static_cast<bf16*>(L.packed[2]);
  g.kT = kT;
  g.qT = qT;
  g.doT = doT;
  g.Dp = L.stat_d;
  g.L2 = L.stat_l2;
  g.dq = L.dq;
  g.dk = L.dk;
  g.dv = L.dv;
  g.B = L.batch;
  g.N = L.seq_len;
  g.Np = L.seq_pad;
  g.H = L.n_heads;
  g.d = L.d_model;
  g.causal = L.causal;
  g.G = L.n_kv_heads;
  g.dkv = L.n_kv_heads * DK;
  g.window = L.window;
  g.chunk = L.chunk;
  g.scale = 1.0f / sqrtf((float)DK);
  g.scale_log2e = kLog2e * g.scale;
  const int bhs = L.batch * L.n_heads;
  const long long stat_threads = (long long)bhs * L.seq_pad * (DK / 8);
  if (mark(L, 0, s, err, n)) return 1;
  hipLaunchKernelGGL(bwd_stats_kernel<DK>, dim3((unsigned)(stat_threads / 256)), dim3(256), 0, s,
                     g.dout, static_cast<const bf16*>(L.out), L.lse, L.stat_d, L.stat_l2, L.batch,
                     L.seq_len, L.seq_pad, L.n_heads);
  if (check_launch("bwd_stats", err, n) || mark(L, 1, s, err, n)) return 1;
  // Q^T, dO^T per (sequence, query head); K^T per (sequence, key/value head)
  TransposeJob job{{g.q, g.dout, nullptr}, {qT, doT, nullptr}};
  hipLaunchKernelGGL(bwd_transpose_kernel, dim3((unsigned)(bhs * (L.seq_pad / 64) * (DK / 64)), 2),
                     dim3(256), 0, s, job, L.seq_len, L.seq_pad, L.n_heads, DK);
  TransposeJob kjob{{g.k, nullptr, nullptr}, {kT, nullptr, nullptr}};
  const int bgs = L.batch * L.n_kv_heads;
  hipLaunchKernelGGL(bwd_transpose_kernel, dim3((unsigned)(bgs * (L.seq_pad / 64) * (DK / 64)), 1),
                     dim3(256), 0, s, kjob, L.seq_len, L.seq_pad, L.n_kv_heads, DK);
  if (check_launch("bwd_transpose", err, n) || mark(L, 2, s, err, n)) return 1;
  // d_k 128: 8 waves share each key/value stage (two per SIMD, 256 query rows);
  // d_k 64: 4 waves, and two workgroups fit one compute unit
  constexpr int DQW = DK == 128 ? 8 : 4;
  // dK / dV at d_k 64: 4 waves and 64-row query stages; at d_k 128 the split kernel
  // of k_attention_bwd_dkv.hip, also one workgroup per 128 keys
  constexpr int DKW = 4, DKQ = 64;
  const int nqb = (L.seq_len + 32 * DQW - 1) / (32 * DQW);
  const int nkb = (L.seq_len + 32 * DKW - 1) / (32 * DKW);
  // masks or grouped key/value heads run the general instances
  const bool general = L.window || L.chunk || L.n_kv_heads != L.n_heads;
  auto kdq = general ? bwd_dq_kernel<DK, DQW, true> : bwd_dq_kernel<DK, DQW, false>;
  // (d_k 128: launch_bwd_dkv128)
  auto kdkv = general ? bwd_dkv_kernel<DK == 128 ? 64 : DK, DKW, DKQ, true>
                      : bwd_dkv_kernel<DK == 128 ? 64 : DK, DKW, DKQ, false>;
  hipLaunchKernelGGL(kdq, dim3(bhs * nqb), dim3(64 * DQW), 0, s, g);
  if (check_launch("bwd_dq", err, n) || mark(L, 3, s, err, n)) return 1;
  if constexpr (DK == 128) {
    static_assert(32 * DKW == 128, "launch_bwd_dkv128 takes one workgroup per 128 keys");
    launch_bwd_dkv128(g, bgs * nkb, general, s);
  } else {
    hipLaunchKernelGGL(kdkv, dim3(bgs * nkb), dim3(64 * DKW), 0, s, g);
  }
  return check_launch("bwd_dkv", err, n) || mark(L, 4, s, err, n);
}

}  // namespace

int launch_attention_bwd(const AttnBwdLaunch& L, void* stream, char* err, size_t n) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (L.d_head == 64) return run_bwd<64>(L, s, err, n);
  if (L.d_head == 128) return run_bwd<128>(L, s, err, n);
  set_err(err, n, "attention backward: head size %s%d unsupported (64 or 128)", "", L.d_head);
  return 1;
}

}  // namespace bpt
