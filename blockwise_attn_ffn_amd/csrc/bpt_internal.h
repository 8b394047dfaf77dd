// Internal interface between the host validation/dispatch layer (bpt_api.cpp,
// plain C++) and the HIP launchers (k_*.hip, bpt_launch.hip). Nothing here is exported.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/bpt.h"

namespace bpt {

// One layer's launch parameters after validation. All pointers are device
// pointers; sizes are in elements unless named *_bytes.
struct LayerLaunch {
  // shape
  int batch, seq_len, d_model, n_heads, d_head, d_ff;
  int n_kv_heads, d_kv, kv_pad;   // key/value heads g, g * d_head, kv_pad_cols(d_kv)
  int block_q, block_kv, causal;
  int window, chunk;   // attention masks on top of the causal one (0: none)
  float ln_eps;
  int compute_f32;   // 1: fp32 operands everywhere; 0: bf16 operands
  int x_f32;         // element type of X: 1 fp32, 0 bf16 (the weights' type otherwise)
  int z_f32;         // element type of Z
  int seq_pad;       // seq_len rounded up to 128: rows per sequence in packed row space
  int split;         // 1: activations carried as bf16 (hi, lo) pairs (precision 1)
  // tensors
  const void* x;
  bpt_layer_weights_t w;
  void* z;
  // workspace carve-up
  int rows_pad;      // batch * seq_pad rounded up to a multiple of 256
  void* xpack;       // LN1(X) as packed B fragments over [rows_pad, d]
  void* q;           // Q as packed B fragments over [rows_pad, d], then O in place
  void* k;           // K: per (sequence, head) packed A fragments [seq_pad keys, d_head]
  void* vt;          // V^T: per (sequence, head) packed A fragments [d_head, seq_pad keys]
  void* wpack;       // W_Q | W_K | W_V, then W_O, W_1, W_2 (epilogue stream, or plain
                     // fragment order for the staged epilogue)
  // staged epilogue (d_model above kFusedMaxWidth): Y fp32 [rows_pad, d] over the
  // K and V^T buffers, and the hidden block [h_rows, d_ff] of packed fragments
  void* ybuf;
  void* hbuf;
  int h_rows;
  // split: the lo halves of LN1(X) / LN2(Y), Q / O, K, V^T and the hidden block
  void* xpack_lo;
  void* q_lo;
  void* k_lo;
  void* vt_lo;
  void* hbuf_lo;
  // optional: 5 hipEvent_t recorded around the 4 kernels (measurement only)
  void* const* events;
  // optional: attention statistic lse [batch, n_heads, seq_len] fp32
  float* lse;
};

// Element counts/byte sizes of the workspace pieces (shared by sizing and carving).
struct WorkspaceLayout {
  size_t xpack_off, q_off, k_off, vt_off, wpack_off, h_off, resid_off, total;
  size_t lo_off[5];   // split: lo halves of xpack, q, k, vt, hidden block
};

// Widest d_model that runs the fused epilogue. Its per-tile fp32 accumulator
// [rows, d_model] lives in registers, which caps the rows per tile (64 at d 1024,
// 32 at d 2048), and each weight fragment it streams feeds rows/32 products: at
// d 2048 that is one product per 1 KB fragment, more weight traffic per CU than
// L2 delivers, and the staged epilogue measured faster. Wider layers, and
// precision 1, use the staged epilogue: one GEMM per step, Y in fp32 and the FFN
// hidden state for a block of rows in the workspace.
constexpr int kFusedMaxWidth = 1024;
inline bool staged_epilogue(int d_model, int split = 0) { return split || d_model > kFusedMaxWidth; }
// Rows of the staged epilogue's hidden block: enough that the W_2 product
// (rows x d_model) spans 512 output tiles of 256 x 256 (2^25 / d_model, a
// multiple of 256), at least 4096, at most the padded rows.
inline size_t hidden_block_rows(int d_model, size_t rows_pad) {
  size_t r = (((size_t)1 << 25) / (size_t)d_model) / 256 * 256;
  if (r < 4096) r = 4096;
  return r < rows_pad ? r : rows_pad;
}

// Attention backward launch parameters after validation (device pointers).
constexpr int kAttnBwdPacked = 3;
struct AttnBwdLaunch {
  int batch, seq_len, d_model, n_heads, d_head, causal;
  int n_kv_heads, window, chunk;   // grouped key/value heads (K, V, dK, dV: n_kv_heads * d_head wide), masks
  int seq_pad;              // seq_len rounded up to 128
  const void *q, *k, *v, *out, *dout;   // bf16 [batch * seq_len, d_model]
  const float* lse;         // [batch, n_heads, seq_len]
  float *dq, *dk, *dv;      // fp32 [batch * seq_len, d_model]
  // workspace carve-up: the row statistics D and lse * log2(e), each fp32
  // [batch * n_heads, seq_pad], then K^T, Q^T and dO^T as bf16 matrix-core
  // fragments over [d_head, tokens] per (sequence, head), [batch * seq_pad, d_model] each
  float* stat_d;
  float* stat_l2;
  void* packed[kAttnBwdPacked];
  // optional: 5 hipEvent_t recorded around the 4 kernels (measurement only)
  void* const* events;
};

// Output features of the K (and of the V) part of the projection product: the
// key/value width rounded up to a whole product tile (256 features for bf16
// operands, 128 for fp32), so that each tile of the QKV product lies inside one
// of Q, K, V (extra features are dropped).
inline int kv_pad_cols(int d_kv, int compute_f32) {
  const int tile = compute_f32 ? 128 : 256;
  return (d_kv + tile - 1) / tile * tile;
}
// Elements of the packed W_Q | W_K | W_V block (kv_pad: kv_pad_cols of d_kv).
inline size_t qkv_pack_elems(int d_model, int kv_pad) {
  return (size_t)(d_model + 2 * kv_pad) * d_model;
}

// Attention forward of one (query shard, key/value shard) pair: row-major bf16 Q,
// K, V in, O (bf16) and lse out; packed: Q (then O), K, V^T copies in the workspace.
struct AttnFwdLaunch {
  int batch, seq_len, seq_pad, d_model, n_heads, d_head, causal;
  const void *q, *k, *v;
  void* o;
  float* lse;
  void* packed[3];
};
int launch_attention_fwd(const AttnFwdLaunch& L, void* stream, char* err, size_t errlen);
int launch_attention_merge(int batch, int seq_len, int n_heads, int d_head, float* o_acc,
                           float* lse_acc, const void* o_part, const float* lse_part, void* stream,
                           char* err, size_t errlen);

// The host (CPU) fused layer: HOST pointers, fp32 arithmetic.
struct HostLaunch {
  int batch, seq_len, d_model, n_heads, n_kv_heads, d_kv, d_ff, block_q, causal, window, chunk;
  float ln_eps;
  int x_f32, w_f32, z_f32;
  const void* x;
  bpt_layer_weights_t w;
  void* z;
  float* kbuf;      // K [batch * seq_len, d_kv]
  float* vbuf;      // V
  float* scratch;   // n_threads x host_scratch_floats
  int n_threads;
};
size_t host_scratch_floats(int d_model, int n_heads, int block_q);
int launch_layer_host(const HostLaunch& L);

// Returns 0 on success, otherwise writes a message into err (errlen bytes).
int launch_layer(const LayerLaunch& L, void* stream, char* err, size_t errlen);

int launch_attention_bwd(const AttnBwdLaunch& L, void* stream, char* err, size_t errlen);

// Whether a kernel instance exists for (d_model, d_head, block sizes, types).
int kernels_support(int d_model, int d_head, int block_q, int block_kv, int compute_f32,
                    int x_f32, int z_f32, int d_ff, int split, char* err, size_t errlen);

}  // namespace bpt
