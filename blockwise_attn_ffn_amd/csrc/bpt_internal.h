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
  // cooperative epilogue (d_model 2048 / 4096): the clusters' exchange regions and
  // the counters (kCoopCtrWords words, zeroed by the launch sequence)
  void* coop_buf;
  void* coop_ctr;
  // optional: 5 hipEvent_t recorded around the 4 kernels (measurement only)
  void* const* events;
  // optional: attention statistic lse [batch, n_heads, seq_len] fp32
  float* lse;
  // optional (attention only, ring share): instead of writing O over Q's copy, merge
  // each finished row into a running state: o_acc fp32 in Q's fragment layout
  // [batch * seq_pad, d], lse_acc [batch, n_heads, seq_len] (natural log)
  float* o_acc;
  float* lse_acc;
};

// Element counts/byte sizes of the workspace pieces (shared by sizing and carving).
struct WorkspaceLayout {
  size_t xpack_off, q_off, k_off, vt_off, wpack_off, h_off, coop_off, coop_ctr_off, resid_off, total;
  size_t lo_off[5];   // split: lo halves of xpack, q, k, vt, hidden block
};

// The cooperative epilogue (k_ffn_coop.hip): clusters of G = d_model / 512
// workgroups on one XCD finish tiles of 128 rows; member g holds output features
// [512 g, 512 g + 512) and computes 256 hidden units of every chunk of 256 G.
constexpr int kCoopRows = 128;
constexpr int kCoopCols = 512;
constexpr int kCoopUnits = 256;
constexpr int kCoopXcds = 8;              // XCDs of the device; workgroups go round-robin
constexpr int kCoopMaxWorkgroups = 256;   // grid bound: sizes the exchange regions
// counter words: per-XCD tickets, the error word, then 4 per cluster (stats, LN2
// operand, hidden chunks, spare)
constexpr int kCoopCtrTickets = 0;
constexpr int kCoopCtrError = 16;
constexpr int kCoopCtrCluster = 32;
constexpr int kCoopCtrWords = kCoopCtrCluster + 4 * kCoopMaxWorkgroups;
// One cluster's exchange region: LN2(Y) of the tile as packed fragments [na
// halves][4 row tiles][d/16 k-steps]; two hidden chunks [2][na][4][hc/16]; the
// per-row partial statistics [2][G][128] (float2); 4 KB aligned. na = 2 with
// bf16 pairs (hi and lo halves), else 1.
struct CoopRegion {
  int d, hc, g, na;
  constexpr size_t a_off() const { return 0; }
  constexpr size_t h_off() const { return (size_t)na * 4 * (d / 16) * 1024; }
  constexpr size_t s_off() const { return h_off() + (size_t)2 * na * 4 * (hc / 16) * 1024; }
  constexpr size_t bytes() const { return (s_off() + (size_t)2 * g * kCoopRows * 8 + 4095) / 4096 * 4096; }
};
inline CoopRegion coop_region(int d_model, int split) {
  const int g = d_model / kCoopCols;
  return CoopRegion{d_model, kCoopUnits * g, g, split ? 2 : 1};
}

// Widest d_model that runs the fused epilogue. Its per-tile fp32 accumulator
// [rows, d_model] lives in registers, which caps the rows per tile (64 at d 1024,
// 32 at d 2048), and each weight fragment it streams feeds rows/32 products: at
// d 2048 that is one product per 1 KB fragment, more weight traffic per CU than
// L2 delivers, and the staged epilogue measured faster. Wider layers, and
// precision 1, use the staged epilogue: one GEMM per step, Y in fp32 and the FFN
// hidden state for a block of rows in the workspace.
constexpr int kFusedMaxWidth = 1024;
// The cooperative epilogue takes d_model 2048 and 4096 in bf16 operands or bf16
// pairs, with d_ff a multiple of its chunk (256 d_model / 512 units).
inline bool coop_epilogue(int d_model, int split, int d_ff) {
  (void)split;
  return (d_model == 2048 || d_model == 4096) && d_ff % (kCoopUnits * (d_model / kCoopCols)) == 0;
}
// The staged epilogue: what neither fused epilogue takes (precision 1 at d_model
// 1024 and below, and wide layers whose d_ff is not a multiple of the chunk).
inline bool staged_epilogue(int d_model, int split, int d_ff) {
  return !coop_epilogue(d_model, split, d_ff) && (split || d_model > kFusedMaxWidth);
}
// W_O, W_1, W_2 in plain fragment order (cooperative or staged epilogue) rather
// than the fused epilogue's per-wave stream.
inline bool plain_epilogue_weights(int d_model, int split, int d_ff) {
  return split || d_model > kFusedMaxWidth;
}
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
  int n_kv_heads;     // 0: n_heads; K and V are [rows, n_kv_heads * d_head]
  int window, chunk;  // masks of the causal setting (0: none)
  const void *q, *k, *v;
  void* o;
  float* lse;
  void* packed[3];
};
int launch_attention_fwd(const AttnFwdLaunch& L, void* stream, char* err, size_t errlen);
int launch_attention_merge(int batch, int seq_len, int n_heads, int d_head, float* o_acc,
                           float* lse_acc, const void* o_part, const float* lse_part, void* stream,
                           char* err, size_t errlen);

// Layer backward (k_layer_bwd.hip) after validation: device pointers; bf16
// buffers are void*. Row-major buffers are [rows, d_model] over the batch *
// seq_len rows; transposed ones ("...t") are [d_model, rows_t].
struct LayerBwdLaunch {
  int batch, seq_len, seq_pad, d_model, n_heads, d_ff, causal, rows;
  int n_kv_heads;     // key/value heads (divides n_heads); K, V are [rows, n_kv_heads * d_head]
  int window, chunk;  // masks of the causal setting (0: none)
  int rows_t;         // row stride of the transposed activations: rows rounded up to 8
  float ln_eps;
  int block_rows;     // FFN rows per block (a multiple of 8 unless it is all the rows)
  int blk_ld;         // row stride of the block's [d_ff, block] buffers (a multiple of 8)
  int wgrad_splits;   // workgroup layers over the rows for the [d, d] weight gradients
  int ffn_splits;     // likewise for dW_1, dW_2 over a block's rows
  int ln_parts;       // workgroups of the LN backward (column partial sums)
  const void* x;      // bf16 [rows, d]
  bpt_layer_weights_t w;
  const float* lse;   // [batch, n_heads, seq_len]
  const float* dz;    // fp32 [rows, d]
  float* dx;          // fp32 [rows, d]
  bpt_layer_grads_t g;
  // workspace (see bpt_api.cpp: bwd_layout for sizes and the reuse of dead buffers)
  void *x1, *q, *k, *v, *attn, *y2, *dzb, *dyb, *da;   // bf16 [rows, d]
  void* dqkvb;          // bf16 [rows, 3d]: dQ | dK | dV per row
  void *x1t, *attnt, *y2t, *dzt, *dyt, *dqt, *dkt, *dvt;                 // bf16 [d, rows_t]
  void *hblk, *dublk;   // bf16 [d_ff, blk_ld]: H^T and dU^T of the block
  float* ublk;          // fp32: U^T of the block in the product kernel's tile fragment order
  void* dub;            // bf16 [block_rows, d_ff]: dU of the block
  void *w1t, *w2t, *wot;   // bf16 weights transposed: [d, d_ff], [d_ff, d], [d, d]
  void* wqkvt;              // bf16 [d, 3d]: W_Q^T | W_K^T | W_V^T
  float *y, *dy2, *dy, *dq, *dk, *dv, *dx1;   // fp32 [rows, d]
  float *stats1, *stats2;   // (mean, rstd) per row: 2 floats each
  float* lse_re;        // the recomputed forward's statistic (not used further)
  float *stat_d, *stat_l2;   // attention backward row statistics [batch * n_heads, seq_pad]
  void* packed[3];      // attention operands in fragment order, [batch * seq_pad, d] bf16 each
  float* partials;      // split-k partial sums: wgrad_splits x [d, d] or ffn_splits x [d, d_ff]
  float* ln_part;       // LN backward column partials: ln_parts x 2 x [d]
};
int launch_layer_bwd(const LayerBwdLaunch& L, void* stream, char* err, size_t errlen);

// Ring Attention, one device's share (k_ring.hip). A key/value shard in the
// attention kernels' fragment layouts: K (rows-A) then V^T (cols-A), each
// [batch * seq_pad, d_model] bf16 on a 256-byte boundary.
struct RingKvLaunch {
  int batch, seq_len, seq_pad, d_model, n_heads, d_head;
  const void *k, *v;   // bf16 row-major [batch * seq_len, d_model]
  void* kv;            // packed shard
  size_t half_bytes;   // bytes of each of the two parts
};
int launch_ring_pack_kv(const RingKvLaunch& L, void* stream, char* err, size_t errlen);

// The share: this device's query shard against n_shards packed key/value shards
// (shard s holds the tokens before this device's own shard for s < own, its own
// shard for s == own); with the causal mask shards after own are not visited and
// shard own is causal, otherwise every shard is unmasked. The steps' results are
// merged in the attention kernel's finalisation into o_acc / lse_acc.
struct RingShareLaunch {
  int batch, seq_len, seq_pad, d_model, n_heads, d_head, causal, n_shards, own;
  const void* q;             // bf16 row-major [batch * seq_len, d_model]
  const void* const* kv;     // HOST array of n_shards device pointers
  size_t kv_half_bytes;
  void* o;                   // bf16 row-major [batch * seq_len, d_model]
  float* lse;                // [batch, n_heads, seq_len]
  void* q_packed;            // workspace: Q in rows-B fragments
  float* o_acc;              // workspace: fp32 in the same layout
  float* lse_acc;            // workspace: [batch, n_heads, seq_len]
};
int launch_ring_share(const RingShareLaunch& L, void* stream, char* err, size_t errlen);

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

// bpt_layer_fwd_noalloc: bytes of the fixed per-device scratch array, and its
// device address on the current device (resolved once per device). Returns 0 on
// success, otherwise writes a message into err.
constexpr size_t kNoallocScratchBytes = BPT_NOALLOC_SCRATCH_BYTES;
int noalloc_scratch(void** ptr, char* err, size_t errlen);

// Returns 0 on success, otherwise writes a message into err (errlen bytes).
int launch_layer(const LayerLaunch& L, void* stream, char* err, size_t errlen);

int launch_attention_bwd(const AttnBwdLaunch& L, void* stream, char* err, size_t errlen);

// Whether every operand the matrix-product kernels take for this shape stays
// under 4 GiB (they address packed operands with 32-bit byte offsets). es is the
// compute type's element size, rows_pad the padded row count of the workspace.
int operands_fit(int d_model, int d_ff, int kv_pad, size_t rows_pad, size_t es, int split,
                 char* err, size_t errlen);

// Whether a kernel instance exists for (d_model, d_head, block sizes, types).
int kernels_support(int d_model, int d_head, int block_q, int block_kv, int compute_f32,
                    int x_f32, int z_f32, int d_ff, int split, char* err, size_t errlen);

}  // namespace bpt
