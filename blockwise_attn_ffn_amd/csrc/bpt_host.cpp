// The fused blockwise layer on the host CPU (fp32 arithmetic), C ABI in
// include/bpt.h (bpt_layer_fwd_host).
//
// "Blockwise Parallel Transformer — BPT" (aicassindra.com), section "On CPUs and
// small language models": on a CPU the [N, 4d] hidden state of an unfused layer
// lives in DRAM and is streamed twice; fused per block of b rows, the [b, 4d] tile
// stays in cache, and b should be the largest whose tile fits the targeted cache
// level. Section "The fused blockwise algorithm" gives the loop: per query block,
// LN1 and Q, an online softmax over key/value blocks, y = x + o/l W_O, then the FFN
// of LN2(y) and the second residual. The outer loop is spread over threads
// (the page: query blocks are independent, across CPU cores too).
//
// Layout of the work: K and V are projected once per sequence (as on the GPU; the
// pseudocode recomputes them in the inner loop, with identical values), then every
// (sequence, query block) is one work item on a thread. Per item the FFN hidden
// state is produced and consumed in chunks of kHidChunk columns: a [b, kHidChunk]
// fp32 tile (256 KB at b = 128) that stays in the core's L2. Every product has the
// form C[i][j] = sum_k A[i][k] B[j][k], because every weight is stored [out, in]
// (k contiguous): gemm_nt below, with B in fp32 or bf16 (widened in registers).
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <thread>
#include <vector>

#include "bpt_internal.h"

namespace bpt {
namespace host {

constexpr int kHidChunk = 512;   // FFN hidden columns per chunk
constexpr int kKvBlock = 64;     // keys per inner-loop block

typedef float v8f __attribute__((vector_size(32)));
typedef uint16_t v8u16 __attribute__((vector_size(16)));
typedef uint32_t v8u32 __attribute__((vector_size(32)));

inline v8f load8(const float* p) {
  v8f v;
  memcpy(&v, p, sizeof(v));
  return v;
}
// 8 bf16 values (raw bits) widened to fp32: the bits move to the high half
inline v8f load8(const uint16_t* p) {
  v8u16 r;
  memcpy(&r, p, sizeof(r));
  const v8u32 w = __builtin_convertvector(r, v8u32) << 16;
  v8f v;
  memcpy(&v, &w, sizeof(v));
  return v;
}
inline float hsum(v8f v) {
  return ((v[0] + v[4]) + (v[1] + v[5])) + ((v[2] + v[6]) + (v[3] + v[7]));
}
inline float to_f32(float x) { return x; }
inline float to_f32(uint16_t b) {
  const uint32_t w = (uint32_t)b << 16;
  float f;
  memcpy(&f, &w, 4);
  return f;
}
inline uint16_t to_bf16(float f) {   // round to nearest even (finite values)
  uint32_t w;
  memcpy(&w, &f, 4);
  w += 0x7FFFu + ((w >> 16) & 1u);
  return (uint16_t)(w >> 16);
}

// C[i * ldc + j] (=, or += with acc) sum_{k < K} A[i * lda + k] B[j * ldb + k] for
// i < M, j < N. K is a multiple of 8. Register block: 4 rows x 2 columns, columns
// outside rows (a pair of B rows in L1 meets every row group of A; chunking K
// so that row groups run outside measured slower: more partial sums and C updates).
template <typename TB>
void gemm_nt(const float* A, int lda, const TB* B, int ldb, float* C, int ldc, int M, int N, int K,
             bool acc) {
  int j = 0;
  for (; j + 2 <= N; j += 2) {
    const TB* b0 = B + (size_t)j * ldb;
    const TB* b1 = b0 + ldb;
    int i = 0;
    for (; i + 4 <= M; i += 4) {
      const float* a0 = A + (size_t)i * lda;
      const float* a1 = a0 + lda;
      const float* a2 = a1 + lda;
      const float* a3 = a2 + lda;
      v8f c00 = {}, c01 = {}, c10 = {}, c11 = {}, c20 = {}, c21 = {}, c30 = {}, c31 = {};
      for (int k = 0; k < K; k += 8) {
        const v8f w0 = load8(b0 + k), w1 = load8(b1 + k);
        const v8f x0 = load8(a0 + k), x1 = load8(a1 + k), x2 = load8(a2 + k), x3 = load8(a3 + k);
        c00 += x0 * w0; c01 += x0 * w1;
        c10 += x1 * w0; c11 += x1 * w1;
        c20 += x2 * w0; c21 += x2 * w1;
        c30 += x3 * w0; c31 += x3 * w1;
      }
      float* c = C + (size_t)i * ldc + j;
      const float r[8] = {hsum(c00), hsum(c01), hsum(c10), hsum(c11),
                          hsum(c20), hsum(c21), hsum(c30), hsum(c31)};
      for (int q = 0; q < 4; ++q) {
        if (acc) {
          c[q * ldc] += r[2 * q];
          c[q * ldc + 1] += r[2 * q + 1];
        } else {
          c[q * ldc] = r[2 * q];
          c[q * ldc + 1] = r[2 * q + 1];
        }
      }
    }
    for (; i < M; ++i) {
      const float* a = A + (size_t)i * lda;
      v8f s0 = {}, s1 = {};
      for (int k = 0; k < K; k += 8) {
        const v8f x = load8(a + k);
        s0 += x * load8(b0 + k);
        s1 += x * load8(b1 + k);
      }
      float* c = C + (size_t)i * ldc + j;
      if (acc) { c[0] += hsum(s0); c[1] += hsum(s1); }
      else { c[0] = hsum(s0); c[1] = hsum(s1); }
    }
  }
  for (; j < N; ++j) {
    const TB* b0 = B + (size_t)j * ldb;
    for (int i = 0; i < M; ++i) {
      const float* a = A + (size_t)i * lda;
      v8f s = {};
      for (int k = 0; k < K; k += 8) s += load8(a + k) * load8(b0 + k);
      float* c = C + (size_t)i * ldc + j;
      if (acc) *c += hsum(s);
      else *c = hsum(s);
    }
  }
}

// LayerNorm of n rows of width d (biased variance, eps inside the root), fp32
template <typename TP>
void layer_norm(const float* x, int n, int d, const TP* g, const TP* b, float eps, float* out) {
  for (int r = 0; r < n; ++r) {
    const float* xr = x + (size_t)r * d;
    float* o = out + (size_t)r * d;
    double mean = 0.0;
    for (int k = 0; k < d; ++k) mean += xr[k];
    mean /= d;
    double var = 0.0;
    for (int k = 0; k < d; ++k) {
      const double c = xr[k] - mean;
      var += c * c;
    }
    var /= d;
    const float rs = (float)(1.0 / sqrt(var + (double)eps)), mu = (float)mean;
    for (int k = 0; k < d; ++k) o[k] = (xr[k] - mu) * rs * to_f32(g[k]) + to_f32(b[k]);
  }
}

inline float gelu_tanh(float u) {
  const float c = 0.7978845608028654f;   // sqrt(2 / pi)
  return 0.5f * u * (1.0f + tanhf(c * (u + 0.044715f * u * u * u)));
}

struct Shape {
  int B, N, d, H, dk, G, dkv, d_ff, bq, causal, window, chunk;
  float eps;
};

// visible keys of query position p: [lo, hi]
inline int key_hi(const Shape& s, int p) {
  if (!s.causal) return s.N - 1;
  if (s.chunk) return std::min((p / s.chunk + 1) * s.chunk, s.N) - 1;
  return p;
}
inline int key_lo(const Shape& s, int p) { return s.window ? std::max(0, p - s.window + 1) : 0; }

// Per-thread scratch (floats).
inline size_t scratch_floats(const Shape& s) {
  const size_t b = s.bq, d = s.d;
  return 6 * b * d                     // x, q (then o), y, ln, zacc, ln1
         + b * kKvBlock                // scores of one head and key block
         + b * kHidChunk               // FFN hidden chunk
         + 2 * b * s.H;                // running max and sum per row and head
}

template <typename TX, typename TW, typename TZ>
struct Layer {
  Shape s;
  const TX* X;
  const TW *ln1_g, *ln1_b, *wq, *wk, *wv, *wo, *ln2_g, *ln2_b, *w1, *w2;
  TZ* Z;
  float *K, *V;   // [B N, dkv]

  void load_rows(size_t r0, int n, float* dst) const {
    for (int r = 0; r < n; ++r)
      for (int k = 0; k < s.d; ++k) dst[(size_t)r * s.d + k] = to_f32(X[(r0 + r) * s.d + k]);
  }

  // K, V of rows [r0, r0 + n)
  void project_kv(size_t r0, int n, float* ws) const {
    float* x = ws;
    float* ln = ws + (size_t)s.bq * s.d;
    load_rows(r0, n, x);
    layer_norm(x, n, s.d, ln1_g, ln1_b, s.eps, ln);
    gemm_nt(ln, s.d, wk, s.d, K + r0 * s.dkv, s.dkv, n, s.dkv, s.d, false);
    gemm_nt(ln, s.d, wv, s.d, V + r0 * s.dkv, s.dkv, n, s.dkv, s.d, false);
  }

  // the fused block: rows [i0, i0 + n) of sequence b
  void block(int bi, int i0, int n, float* ws) const {
    const size_t bq = s.bq, d = s.d;
    float* x = ws;
    float* q = x + bq * d;      // Q, then the attention output o (per head, in place)
    float* y = q + bq * d;
    float* ln = y + bq * d;
    float* zacc = ln + bq * d;
    float* ln1 = zacc + bq * d;
    float* sc = ln1 + bq * d;   // [n, kKvBlock]
    float* hid = sc + bq * kKvBlock;
    float* mrun = hid + bq * kHidChunk;
    float* lrun = mrun + bq * s.H;
    const size_t r0 = (size_t)bi * s.N + i0;
    load_rows(r0, n, x);
    layer_norm(x, n, s.d, ln1_g, ln1_b, s.eps, ln1);
    gemm_nt(ln1, s.d, wq, s.d, q, s.d, n, s.d, s.d, false);
    const float scale = 1.0f / sqrtf((float)s.dk);
    const float* Kb = K + (size_t)bi * s.N * s.dkv;
    const float* Vb = V + (size_t)bi * s.N * s.dkv;
    const int kfirst = key_lo(s, i0) / kKvBlock * kKvBlock, klast = key_hi(s, i0 + n - 1);
    float* o = y;   // per-head accumulators [n, d] (y is free until W_O)
    for (int h = 0; h < s.H; ++h) {
      const int kvh = h / (s.H / s.G);
      float* m = mrun + (size_t)h * bq;
      float* l = lrun + (size_t)h * bq;
      for (int r = 0; r < n; ++r) {
        m[r] = -INFINITY;
        l[r] = 0.f;
        memset(o + (size_t)r * d + h * s.dk, 0, sizeof(float) * s.dk);
      }
      for (int j0 = kfirst; j0 <= klast; j0 += kKvBlock) {
        const int nk = std::min(kKvBlock, s.N - j0);
        gemm_nt(q + h * s.dk, s.d, Kb + (size_t)j0 * s.dkv + kvh * s.dk, s.dkv, sc, kKvBlock, n, nk,
                s.dk, false);
        for (int r = 0; r < n; ++r) {
          const int p = i0 + r, hi = key_hi(s, p) - j0, lo = key_lo(s, p) - j0;
          float* sr = sc + (size_t)r * kKvBlock;
          float mx = -INFINITY;
          for (int c = 0; c < nk; ++c) {
            sr[c] = (c > hi || c < lo) ? -INFINITY : sr[c] * scale;
            mx = std::max(mx, sr[c]);
          }
          if (mx == -INFINITY) continue;                  // no key of this block visible
          const float mn = std::max(m[r], mx);
          const float alpha = m[r] == -INFINITY ? 0.f : expf(m[r] - mn);
          float* orow = o + (size_t)r * d + h * s.dk;
          if (alpha != 1.f)
            for (int k = 0; k < s.dk; ++k) orow[k] *= alpha;
          float sum = 0.f;
          for (int c = 0; c < nk; ++c) {
            const float e = expf(sr[c] - mn);             // exp(-inf) = 0 for masked keys
            sum += e;
            if (e != 0.f) {
              const float* v = Vb + (size_t)(j0 + c) * s.dkv + kvh * s.dk;
              for (int k = 0; k < s.dk; ++k) orow[k] += e * v[k];
            }
          }
          l[r] = alpha * l[r] + sum;
          m[r] = mn;
        }
      }
    }
    // O = o / l, heads concatenated (into q's space)
    for (int r = 0; r < n; ++r)
      for (int h = 0; h < s.H; ++h) {
        const float inv = 1.0f / lrun[(size_t)h * bq + r];
        const float* orow = o + (size_t)r * d + h * s.dk;
        float* dst = q + (size_t)r * d + h * s.dk;
        for (int k = 0; k < s.dk; ++k) dst[k] = orow[k] * inv;
      }
    // y = x + O W_O;  Z = y + GELU(LN2(y) W_1) W_2, the hidden state in chunks
    gemm_nt(q, s.d, wo, s.d, y, s.d, n, s.d, s.d, false);
    for (size_t e = 0; e < (size_t)n * d; ++e) y[e] += x[e];
    layer_norm(y, n, s.d, ln2_g, ln2_b, s.eps, ln);
    memcpy(zacc, y, sizeof(float) * n * d);
    for (int c0 = 0; c0 < s.d_ff; c0 += kHidChunk) {
      const int hc = std::min(kHidChunk, s.d_ff - c0);
      gemm_nt(ln, s.d, w1 + (size_t)c0 * s.d, s.d, hid, kHidChunk, n, hc, s.d, false);
      for (int r = 0; r < n; ++r)
        for (int c = 0; c < hc; ++c) hid[(size_t)r * kHidChunk + c] = gelu_tanh(hid[(size_t)r * kHidChunk + c]);
      gemm_nt(hid, kHidChunk, w2 + c0, s.d_ff, zacc, s.d, n, s.d, hc, true);
    }
    for (int r = 0; r < n; ++r)
      for (int k = 0; k < s.d; ++k) {
        const float v = zacc[(size_t)r * d + k];
        if constexpr (sizeof(TZ) == 2) Z[(r0 + r) * d + k] = to_bf16(v);
        else Z[(r0 + r) * d + k] = v;
      }
  }
};

// Run f(item, thread) for items [0, n) on n_threads threads.
template <typename F>
void parallel_for(long long n, int n_threads, F f) {
  std::atomic<long long> next{0};
  auto worker = [&](int t) {
    for (long long i = next++; i < n; i = next++) f(i, t);
  };
  std::vector<std::thread> pool;
  for (int t = 1; t < n_threads; ++t) pool.emplace_back(worker, t);
  worker(0);
  for (auto& th : pool) th.join();
}

template <typename TX, typename TW, typename TZ>
void run(const HostLaunch& L) {
  Layer<TX, TW, TZ> ly;
  ly.s = Shape{L.batch, L.seq_len, L.d_model, L.n_heads, L.d_model / L.n_heads, L.n_kv_heads,
               L.d_kv, L.d_ff, L.block_q, L.causal, L.window, L.chunk, L.ln_eps};
  ly.X = static_cast<const TX*>(L.x);
  const bpt_layer_weights_t& w = L.w;
  ly.ln1_g = static_cast<const TW*>(w.ln1_g);
  ly.ln1_b = static_cast<const TW*>(w.ln1_b);
  ly.wq = static_cast<const TW*>(w.w_q);
  ly.wk = static_cast<const TW*>(w.w_k);
  ly.wv = static_cast<const TW*>(w.w_v);
  ly.wo = static_cast<const TW*>(w.w_o);
  ly.ln2_g = static_cast<const TW*>(w.ln2_g);
  ly.ln2_b = static_cast<const TW*>(w.ln2_b);
  ly.w1 = static_cast<const TW*>(w.w_1);
  ly.w2 = static_cast<const TW*>(w.w_2);
  ly.Z = static_cast<TZ*>(L.z);
  ly.K = L.kbuf;
  ly.V = L.vbuf;
  const Shape& s = ly.s;
  const size_t per = scratch_floats(s);
  const long long rows = (long long)s.B * s.N;
  const long long kv_items = (rows + s.bq - 1) / s.bq;
  parallel_for(kv_items, L.n_threads, [&](long long it, int t) {
    const size_t r0 = (size_t)it * s.bq;
    ly.project_kv(r0, (int)std::min<long long>(s.bq, rows - (long long)r0), L.scratch + per * t);
  });
  const int nqb = (s.N + s.bq - 1) / s.bq;
  parallel_for((long long)s.B * nqb, L.n_threads, [&](long long it, int t) {
    const int bi = (int)(it / nqb), qb = (int)(it % nqb);
    const int i0 = qb * s.bq;
    ly.block(bi, i0, std::min(s.bq, s.N - i0), L.scratch + per * t);
  });
}

}  // namespace host

size_t host_scratch_floats(int d_model, int n_heads, int block_q) {
  host::Shape s{};
  s.d = d_model;
  s.H = n_heads;
  s.bq = block_q;
  return host::scratch_floats(s);
}

int launch_layer_host(const HostLaunch& L) {
  const bool xf = L.x_f32, wf = L.w_f32, zf = L.z_f32;
  using bf = uint16_t;
  if (xf && wf && zf) host::run<float, float, float>(L);
  else if (xf && wf && !zf) host::run<float, float, bf>(L);
  else if (!xf && !wf && zf) host::run<bf, bf, float>(L);
  else if (!xf && !wf && !zf) host::run<bf, bf, bf>(L);
  else if (xf && !wf && zf) host::run<float, bf, float>(L);
  else if (xf && !wf && !zf) host::run<float, bf, bf>(L);
  else return 1;
  return 0;
}

}  // namespace bpt
