// One device's share of Ring Attention (gfx950).
//
// "Blockwise Parallel Transformer — BPT" (aicassindra.com), section "BPT and Ring
// Attention": the sequence is sharded across devices, each device keeps its query
// shard, and key/value shards travel around a ring until every query has met every
// key; BPT's inner loop already consumes K/V a block at a time, so only where the
// next block comes from changes. On one device a step is attention of the local
// query shard against the shard that arrived (causal within the device's own shard,
// unmasked against earlier shards, nothing against later ones), and the steps'
// normalised outputs are combined through their saved statistics:
//   lse = ln(e^lse_a + e^lse_b),   O = e^(lse_a - lse) O_a + e^(lse_b - lse) O_b,
// the same rescaling the online softmax applies between key/value blocks.
//
// attention_fwd: row-major Q, K, V (bf16) are copied into the attention kernel's
// fragment layouts, the layer's attention kernel runs on them (writing O over Q's
// copy and lse), and O is copied back to row-major. merge: the running state (fp32)
// absorbs one step's (O, lse).
#include "attn_pack.hpp"
#include "bpt_device.hpp"
#include "bpt_launch.hpp"

namespace bpt {

// Running state update, one thread per (row, head): acc <- merge(acc, part).
__global__ __launch_bounds__(256) void attn_merge_kernel(float* __restrict__ o_acc,
                                                         float* __restrict__ lse_acc,
                                                         const bf16* __restrict__ o_part,
                                                         const float* __restrict__ lse_part, int B,
                                                         int N, int H, int dk) {
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;   // ((b H + h) N + pos)
  if (t >= (long long)B * H * N) return;
  const int pos = (int)(t % N);
  const long long bh = t / N;
  const int h = (int)(bh % H), b = (int)(bh / H);
  const float la = lse_acc[t], lb = lse_part[t];
  const float m = fmaxf(la, lb);                     // lb is finite: a row sees its own key
  const float lse = m + logf(expf(la - m) + expf(lb - m));
  const float wa = expf(la - lse), wb = expf(lb - lse);   // wa = 0 while acc is empty (-inf)
  const size_t off = ((size_t)b * N + pos) * (size_t)(H * dk) + (size_t)h * dk;
  for (int j = 0; j < dk; j += 8) {
    float a[8], p[8];
    load8_f32(o_acc + off + j, a);
    load8_f32(o_part + off + j, p);
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = wa == 0.f ? wb * p[e] : fmaf(wa, a[e], wb * p[e]);
    store8_f32(o_acc + off + j, a);
  }
  lse_acc[t] = lse;
}

int launch_attention_fwd(const AttnFwdLaunch& A, void* stream, char* err, size_t n) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int B = A.batch, N = A.seq_len, Np = A.seq_pad, H = A.n_heads, dk = A.d_head, d = A.d_model;
  const int G = A.n_kv_heads > 0 ? A.n_kv_heads : H, dkv = G * dk;
  if (d != H * dk || Np % 128 != 0 || Np < N || N < 1 || H % G != 0) {
    set_err(err, n, "attention forward: inconsistent launch shape%s (seq_pad %d)", "", Np);
    return 1;
  }
  bf16* qp = static_cast<bf16*>(A.packed[0]);
  bf16* kp = static_cast<bf16*>(A.packed[1]);
  bf16* vtp = static_cast<bf16*>(A.packed[2]);
  const long long chunks = (long long)B * Np * (d / 8), kv_chunks = (long long)B * Np * (dkv / 8);
  hipLaunchKernelGGL(pack_rows_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, s,
                     static_cast<const bf16*>(A.q), qp, (int)kRowsB, B, N, Np, H, dk);
  // K and V^T per key/value head
  hipLaunchKernelGGL(pack_rows_kernel, dim3((unsigned)((kv_chunks + 255) / 256)), dim3(256), 0, s,
                     static_cast<const bf16*>(A.k), kp, (int)kRowsA, B, N, Np, G, dk);
  TransposeJob job{{static_cast<const bf16*>(A.v), nullptr, nullptr}, {vtp, nullptr, nullptr}};
  hipLaunchKernelGGL(bwd_transpose_kernel, dim3((unsigned)(B * G * (Np / 64) * (dk / 64)), 1),
                     dim3(256), 0, s, job, N, Np, G, dk);
  if (check_launch("attention_fwd pack", err, n)) return 1;
  // the layer's attention kernels on the packed operands (block sizes of the
  // tuned path: 128-row query blocks; 64-key blocks at d_k 128, 128 at d_k 64)
  LayerLaunch L{};
  L.batch = B;
  L.seq_len = N;
  L.seq_pad = Np;
  L.d_model = d;
  L.n_heads = H;
  L.n_kv_heads = G;
  L.d_kv = dkv;
  L.window = A.window;
  L.chunk = A.chunk;
  L.d_head = dk;
  L.block_q = 128;
  L.block_kv = dk == 128 ? 64 : 128;
  L.causal = A.causal;
  L.q = qp;
  L.k = kp;
  L.vt = vtp;
  L.lse = A.lse;
  if (launch_attention(L, s, err, n)) return 1;
  const long long out_chunks = (long long)B * N * (d / 8);
  hipLaunchKernelGGL(unpack_rows_kernel, dim3((unsigned)((out_chunks + 255) / 256)), dim3(256), 0, s,
                     qp, static_cast<bf16*>(A.o), B, N, Np, d);
  return check_launch("attention_fwd unpack", err, n);
}

// The share's running statistic starts at -inf (no key seen).
__global__ __launch_bounds__(256) void ring_fill_kernel(float* __restrict__ p, long long n, float v) {
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t < n) p[t] = v;
}

// The share's result: fp32 rows-B fragments [B Np, d] -> bf16 row-major [B N, d].
__global__ __launch_bounds__(256) void ring_unpack_kernel(const float* __restrict__ src,
                                                          bf16* __restrict__ dst, int B, int N, int Np,
                                                          int d) {
  const int cpr = d / 8;
  const long long s = (long long)blockIdx.x * 256 + threadIdx.x;
  if (s >= (long long)B * N * cpr) return;
  const long long row = s / cpr;
  const int col = (int)(s - row * cpr) * 8;
  const int b = (int)(row / N), pos = (int)(row - (long long)b * N);
  const long long prow = (long long)b * Np + pos;
  const size_t frag = (size_t)(prow >> 5) * (d / 16) + (col >> 4);
  const int slot = 32 * ((col >> 3) & 1) + (int)(prow & 31);
  float v[8];
  load8_f32(src + frag * kFragElems + slot * 8, v);
  store8_f32(dst + row * d + col, v);
}

int launch_ring_pack_kv(const RingKvLaunch& A, void* stream, char* err, size_t n) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int B = A.batch, N = A.seq_len, Np = A.seq_pad, dk = A.d_head, H = A.n_heads, d = A.d_model;
  if (d != H * dk || Np % 128 != 0 || Np < N || N < 1) {
    set_err(err, n, "ring key/value packing: inconsistent shape%s (seq_pad %d)", "", Np);
    return 1;
  }
  bf16* kp = static_cast<bf16*>(A.kv);
  bf16* vtp = reinterpret_cast<bf16*>(static_cast<char*>(A.kv) + A.half_bytes);
  const long long chunks = (long long)B * Np * (d / 8);
  hipLaunchKernelGGL(pack_rows_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, s,
                     static_cast<const bf16*>(A.k), kp, (int)kRowsA, B, N, Np, H, dk);
  TransposeJob job{{static_cast<const bf16*>(A.v), nullptr, nullptr}, {vtp, nullptr, nullptr}};
  hipLaunchKernelGGL(bwd_transpose_kernel, dim3((unsigned)(B * H * (Np / 64) * (dk / 64)), 1), dim3(256), 0, s,
                     job, N, Np, H, dk);
  return check_launch("ring_pack_kv", err, n);
}

int launch_ring_share(const RingShareLaunch& A, void* stream, char* err, size_t n) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int B = A.batch, N = A.seq_len, Np = A.seq_pad, H = A.n_heads, dk = A.d_head, d = A.d_model;
  if (d != H * dk || Np % 128 != 0 || Np < N || N < 1 || A.n_shards < 1 || A.own < 0 ||
      A.own >= A.n_shards) {
    set_err(err, n, "ring share: inconsistent shape%s (seq_pad %d)", "", Np);
    return 1;
  }
  // this device's queries, packed once for every step
  const long long chunks = (long long)B * Np * (d / 8);
  hipLaunchKernelGGL(pack_rows_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, s,
                     static_cast<const bf16*>(A.q), static_cast<bf16*>(A.q_packed), (int)kRowsB, B, N, Np, H,
                     dk);
  const long long nl = (long long)B * H * N;
  hipLaunchKernelGGL(ring_fill_kernel, dim3((unsigned)((nl + 255) / 256)), dim3(256), 0, s, A.lse_acc, nl,
                     -INFINITY);
  if (check_launch("ring_share prep", err, n)) return 1;
  for (int sh = 0; sh < A.n_shards; ++sh) {
    if (A.causal && sh > A.own) continue;   // wholly in these queries' future
    LayerLaunch L{};
    L.batch = B;
    L.seq_len = N;
    L.seq_pad = Np;
    L.d_model = d;
    L.n_heads = H;
    L.n_kv_heads = H;
    L.d_kv = d;
    L.d_head = dk;
    L.block_q = 128;
    L.block_kv = dk == 128 ? 64 : 128;
    L.causal = A.causal && sh == A.own;
    L.q = A.q_packed;
    L.k = const_cast<void*>(A.kv[sh]);   // read only by the attention kernels
    L.vt = const_cast<char*>(static_cast<const char*>(A.kv[sh])) + A.kv_half_bytes;
    L.o_acc = A.o_acc;
    L.lse_acc = A.lse_acc;
    if (launch_attention(L, s, err, n)) return 1;
  }
  const long long out_chunks = (long long)B * N * (d / 8);
  hipLaunchKernelGGL(ring_unpack_kernel, dim3((unsigned)((out_chunks + 255) / 256)), dim3(256), 0, s, A.o_acc,
                     static_cast<bf16*>(A.o), B, N, Np, d);
  if (check_launch("ring_share unpack", err, n)) return 1;
  const hipError_t e = hipMemcpyAsync(A.lse, A.lse_acc, (size_t)nl * sizeof(float), hipMemcpyDeviceToDevice, s);
  if (e != hipSuccess) {
    set_err(err, n, "ring share: lse copy: %s", hipGetErrorString(e));
    return 1;
  }
  return 0;
}

int launch_attention_merge(int B, int N, int H, int dk, float* o_acc, float* lse_acc,
                           const void* o_part, const float* lse_part, void* stream, char* err,
                           size_t n) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const long long t = (long long)B * H * N;
  hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)((t + 255) / 256)), dim3(256), 0, s, o_acc,
                     lse_acc, static_cast<const bf16*>(o_part), lse_part, B, N, H, dk);
  return check_launch("attention_merge", err, n);
}

}  // namespace bpt
