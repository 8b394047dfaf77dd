// Host side of the C ABI declared in include/bpt.h: validation, workspace
// sizing and carving, and the per-layer / per-stack launch sequence.
// Plain C++ (no HIP headers): the launches themselves live in the k_*.hip units.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "bpt_internal.h"

namespace {

thread_local char g_err[512] = "";

bpt_status_t fail(bpt_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

constexpr size_t kAlign = 256;
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

size_t esize(int dtype) { return dtype == BPT_F32 ? 4 : 2; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

size_t seq_pad_of(const bpt_layer_desc_t* d) { return round_up((size_t)d->seq_len, 128); }
int kv_heads(const bpt_layer_desc_t* d) { return d->n_kv_heads ? d->n_kv_heads : d->n_heads; }
size_t kv_width(const bpt_layer_desc_t* d) {
  return (size_t)kv_heads(d) * (size_t)(d->d_model / d->n_heads);
}
size_t rows_pad_of(const bpt_layer_desc_t* d) { return round_up((size_t)d->batch * seq_pad_of(d), 256); }

// Layout of the layer workspace, plus the stack's fp32 residual buffer.
bpt::WorkspaceLayout layout(const bpt_layer_desc_t* d, bool stack_resid) {
  bpt::WorkspaceLayout L{};
  const size_t rows = (size_t)d->batch * d->seq_len;
  const size_t es = esize(d->dtype);
  const size_t dm = d->d_model, df = d->d_ff;
  const size_t rp = rows_pad_of(d);
  const bool split = d->precision == 1;
  const bool staged = bpt::staged_epilogue(d->d_model, split, d->d_ff);
  const bool coop = bpt::coop_epilogue(d->d_model, split, d->d_ff);
  const size_t dkv = kv_width(d);
  // K and V^T cover rows_pad rows on the staged path, so that the fp32 Y [rows_pad, d]
  // fits over them once attention is done
  const size_t used = staged ? rp : (size_t)d->batch * seq_pad_of(d);
  size_t off = 0;
  L.xpack_off = off;  // LN1(X), packed
  off = round_up(off + rp * dm * es, kAlign);
  L.q_off = off;      // Q, then O, packed
  off = round_up(off + rp * dm * es, kAlign);
  L.k_off = off;      // K, packed per (sequence, key/value head)
  off = round_up(off + used * dkv * es, kAlign);
  L.vt_off = off;     // V^T, packed per (sequence, key/value head)
  off = round_up(off + used * dkv * es, kAlign);
  if (staged && off - L.k_off < rp * dm * 4)   // fewer key/value heads: room for Y
    off = L.k_off + round_up(rp * dm * 4, kAlign);
  L.wpack_off = off;  // W_Q, W_K, W_V (padded), W_O, W_1, W_2 back to back, fragment order
  const int kvp = bpt::kv_pad_cols((int)dkv, d->dtype == BPT_F32);
  off = round_up(off + (bpt::qkv_pack_elems(d->d_model, kvp) + dm * dm + 2 * df * dm) * es, kAlign);
  L.h_off = off;      // staged epilogue: hidden block [hidden_block_rows, d_ff]
  const size_t hr = bpt::hidden_block_rows(d->d_model, rp);
  if (staged) off = round_up(off + hr * df * es, kAlign);
  L.coop_off = off;   // cooperative epilogue: the clusters' exchange regions, then counters
  if (coop) {
    const size_t clusters = bpt::kCoopMaxWorkgroups / (d->d_model / bpt::kCoopCols);
    off = round_up(off + clusters * bpt::coop_region(d->d_model, split).bytes(), kAlign);
    L.coop_ctr_off = off;
    off = round_up(off + (size_t)bpt::kCoopCtrWords * 4, kAlign);
  }
  if (split) {        // lo halves, same shapes as the hi ones
    const size_t sizes[5] = {rp * dm * es, rp * dm * es, used * dkv * es, used * dkv * es,
                             staged ? hr * df * es : 0};
    for (int i = 0; i < 5; ++i) {
      L.lo_off[i] = off;
      off = round_up(off + sizes[i], kAlign);
    }
  }
  L.resid_off = off;
  if (stack_resid) off = round_up(off + rows * dm * 4, kAlign);
  L.total = off;
  return L;
}

bool is_empty(const bpt_layer_desc_t* d) { return d->batch == 0 || d->seq_len == 0; }

// Shape/option validation shared by both entry points (no pointers).
bpt_status_t validate_desc(const bpt_layer_desc_t* d) {
  if (!d) return fail(BPT_ERR_NULL, "desc is NULL");
  if (d->batch < 0 || d->seq_len < 0) return fail(BPT_ERR_SHAPE, "batch and seq_len must be >= 0");
  if (d->d_model <= 0 || d->n_heads <= 0 || d->d_ff <= 0)
    return fail(BPT_ERR_SHAPE, "d_model, n_heads and d_ff must be > 0");
  if (d->d_model % d->n_heads != 0)
    return fail(BPT_ERR_SHAPE, "d_model %d is not a multiple of n_heads %d", d->d_model, d->n_heads);
  if (d->block_q <= 0 || d->block_kv <= 0) return fail(BPT_ERR_SHAPE, "block sizes must be > 0");
  if (d->causal != 0 && d->causal != 1) return fail(BPT_ERR_SHAPE, "causal must be 0 or 1");
  if (d->window < 0 || d->chunk < 0) return fail(BPT_ERR_SHAPE, "window and chunk must be >= 0");
  if ((d->window || d->chunk) && !d->causal)
    return fail(BPT_ERR_SHAPE, "window and chunk apply to the causal mask only");
  if (d->window && d->chunk) return fail(BPT_ERR_SHAPE, "window and chunk cannot be combined");
  if (d->n_kv_heads < 0 || (d->n_kv_heads && d->n_heads % d->n_kv_heads != 0))
    return fail(BPT_ERR_SHAPE, "n_kv_heads %d must be 0 or divide n_heads %d", d->n_kv_heads,
                d->n_heads);
  if (!(d->ln_eps > 0.0f) || !isfinite(d->ln_eps))
    return fail(BPT_ERR_SHAPE, "ln_eps must be finite and > 0");
  if ((d->dtype != BPT_F32 && d->dtype != BPT_BF16) ||
      (d->out_dtype != BPT_F32 && d->out_dtype != BPT_BF16))
    return fail(BPT_ERR_SHAPE, "dtype / out_dtype must be BPT_F32 or BPT_BF16");
  if (d->act != 0) return fail(BPT_ERR_UNSUPPORTED, "act %d unsupported (0 = GELU tanh)", d->act);
  if (d->precision != 0 && d->precision != 1)
    return fail(BPT_ERR_SHAPE, "precision must be 0 (bf16) or 1 (bf16 pairs)");
  if ((int64_t)d->batch * d->seq_len > (int64_t)INT32_MAX - 1024)
    return fail(BPT_ERR_SHAPE, "batch * seq_len exceeds the 32-bit row index range");
  char msg[256] = "";
  if (!bpt::kernels_support(d->d_model, d->d_model / d->n_heads, d->block_q, d->block_kv,
                            d->dtype == BPT_F32, 0, d->out_dtype == BPT_F32, d->d_ff,
                            d->precision == 1, msg, sizeof(msg)))
    return fail(BPT_ERR_UNSUPPORTED, "%s", msg);
  // The matrix-product kernels address each packed operand with 32-bit byte
  // offsets: every operand they are given must stay under 4 GiB.
  const int kvp = bpt::kv_pad_cols((int)kv_width(d), d->dtype == BPT_F32);
  if (!bpt::operands_fit(d->d_model, d->d_ff, kvp, rows_pad_of(d), esize(d->dtype),
                         d->precision == 1, msg, sizeof(msg)))
    return fail(BPT_ERR_UNSUPPORTED, "%s", msg);
  return BPT_OK;
}

bpt_status_t validate_weights(const bpt_layer_weights_t* w, int idx) {
  if (!w) return fail(BPT_ERR_NULL, "weights[%d] is NULL", idx);
  const void* p[10] = {w->ln1_g, w->ln1_b, w->w_q, w->w_k, w->w_v,
                       w->w_o,   w->ln2_g, w->ln2_b, w->w_1, w->w_2};
  static const char* names[10] = {"ln1_g", "ln1_b", "w_q", "w_k", "w_v",
                                  "w_o",   "ln2_g", "ln2_b", "w_1", "w_2"};
  for (int i = 0; i < 10; ++i) {
    if (!p[i]) return fail(BPT_ERR_NULL, "weights[%d].%s is NULL", idx, names[i]);
    if (!aligned16(p[i]))
      return fail(BPT_ERR_ALIGN, "weights[%d].%s is not 16-byte aligned", idx, names[i]);
  }
  return BPT_OK;
}

bpt_status_t validate_buffers(const bpt_layer_desc_t* d, const void* X, const void* Z,
                              void* ws, size_t ws_bytes, size_t need) {
  if (!X) return fail(BPT_ERR_NULL, "X is NULL");
  if (!Z) return fail(BPT_ERR_NULL, "Z is NULL");
  if (!aligned16(X)) return fail(BPT_ERR_ALIGN, "X is not 16-byte aligned");
  if (!aligned16(Z)) return fail(BPT_ERR_ALIGN, "Z is not 16-byte aligned");
  if (ws_bytes < need)
    return fail(BPT_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
  if (need > 0 && !ws) return fail(BPT_ERR_NULL, "workspace is NULL");
  if (ws && !aligned16(ws)) return fail(BPT_ERR_ALIGN, "workspace is not 16-byte aligned");
  const size_t rows = (size_t)d->batch * d->seq_len;
  const size_t xb = rows * d->d_model * esize(d->dtype);
  const size_t zb = rows * d->d_model * esize(d->out_dtype);
  if (overlap(X, xb, Z, zb)) return fail(BPT_ERR_ALIAS, "X and Z overlap");
  if (overlap(ws, need, X, xb)) return fail(BPT_ERR_ALIAS, "workspace overlaps X");
  if (overlap(ws, need, Z, zb)) return fail(BPT_ERR_ALIAS, "workspace overlaps Z");
  return BPT_OK;
}

bpt::LayerLaunch make_launch(const bpt_layer_desc_t* d, const bpt::WorkspaceLayout& L, void* ws) {
  bpt::LayerLaunch p{};
  p.batch = d->batch;
  p.seq_len = d->seq_len;
  p.d_model = d->d_model;
  p.n_heads = d->n_heads;
  p.d_head = d->d_model / d->n_heads;
  p.d_ff = d->d_ff;
  p.n_kv_heads = kv_heads(d);
  p.d_kv = (int)kv_width(d);
  p.kv_pad = bpt::kv_pad_cols(p.d_kv, d->dtype == BPT_F32);
  p.block_q = d->block_q;
  p.block_kv = d->block_kv;
  p.causal = d->causal;
  p.window = d->window;
  p.chunk = d->chunk;
  p.ln_eps = d->ln_eps;
  p.compute_f32 = d->dtype == BPT_F32;
  p.seq_pad = (int)seq_pad_of(d);
  p.split = d->precision == 1;
  char* base = static_cast<char*>(ws);
  p.rows_pad = (int)rows_pad_of(d);
  p.xpack = base + L.xpack_off;
  p.q = base + L.q_off;
  p.k = base + L.k_off;
  p.vt = base + L.vt_off;
  p.wpack = base + L.wpack_off;
  if (bpt::coop_epilogue(d->d_model, p.split, d->d_ff)) {
    p.coop_buf = base + L.coop_off;
    p.coop_ctr = base + L.coop_ctr_off;
  }
  if (bpt::staged_epilogue(d->d_model, p.split, d->d_ff)) {
    p.ybuf = base + L.k_off;
    p.hbuf = base + L.h_off;
    p.h_rows = (int)bpt::hidden_block_rows(p.d_model, (size_t)p.rows_pad);
  }
  if (p.split) {
    p.xpack_lo = base + L.lo_off[0];
    p.q_lo = base + L.lo_off[1];
    p.k_lo = base + L.lo_off[2];
    p.vt_lo = base + L.lo_off[3];
    p.hbuf_lo = base + L.lo_off[4];
  }
  return p;
}

bpt_status_t run(bpt::LayerLaunch& p, void* stream) {
  char msg[256] = "";
  if (bpt::launch_layer(p, stream, msg, sizeof(msg))) return fail(BPT_ERR_HIP, "%s", msg);
  return BPT_OK;
}

// One layer call: validation, launch record, launch. lse (optional) receives the
// attention statistic [batch, n_heads, seq_len] fp32 and must overlap no other buffer.
bpt_status_t layer_call(const bpt_layer_desc_t* desc, const void* X,
                        const bpt_layer_weights_t* weights, void* Z, float* lse, void* workspace,
                        size_t workspace_bytes, void* hip_stream, void* const* events) {
  bpt_status_t st = validate_desc(desc);
  if (st != BPT_OK) return st;
  if (is_empty(desc)) return BPT_OK;
  if ((st = validate_weights(weights, 0)) != BPT_OK) return st;
  const bpt::WorkspaceLayout L = layout(desc, false);
  if ((st = validate_buffers(desc, X, Z, workspace, workspace_bytes, L.total)) != BPT_OK) return st;
  if (lse) {
    const size_t rows = (size_t)desc->batch * desc->seq_len;
    const size_t lb = (size_t)desc->n_heads * rows * sizeof(float);
    if (overlap(lse, lb, X, rows * desc->d_model * esize(desc->dtype)))
      return fail(BPT_ERR_ALIAS, "lse overlaps X");
    if (overlap(lse, lb, Z, rows * desc->d_model * esize(desc->out_dtype)))
      return fail(BPT_ERR_ALIAS, "lse overlaps Z");
    if (overlap(lse, lb, workspace, L.total)) return fail(BPT_ERR_ALIAS, "lse overlaps the workspace");
  }
  bpt::LayerLaunch p = make_launch(desc, L, workspace);
  p.x = X;
  p.x_f32 = desc->dtype == BPT_F32;
  p.z = Z;
  p.z_f32 = desc->out_dtype == BPT_F32;
  p.w = *weights;
  p.events = events;
  p.lse = lse;
  return run(p, hip_stream);
}


// ---------------------------------------------------------------------------
// Attention backward
// ---------------------------------------------------------------------------

bool attn_empty(const bpt_attn_desc_t* d) { return d->batch == 0 || d->seq_len == 0; }

bpt_status_t validate_attn_desc(const bpt_attn_desc_t* d) {
  if (!d) return fail(BPT_ERR_NULL, "desc is NULL");
  if (d->batch < 0 || d->seq_len < 0) return fail(BPT_ERR_SHAPE, "batch and seq_len must be >= 0");
  if (d->d_model <= 0 || d->n_heads <= 0) return fail(BPT_ERR_SHAPE, "d_model and n_heads must be > 0");
  if (d->d_model % d->n_heads != 0)
    return fail(BPT_ERR_SHAPE, "d_model %d is not a multiple of n_heads %d", d->d_model, d->n_heads);
  if (d->causal != 0 && d->causal != 1) return fail(BPT_ERR_SHAPE, "causal must be 0 or 1");
  if (d->dtype != BPT_F32 && d->dtype != BPT_BF16)
    return fail(BPT_ERR_SHAPE, "dtype must be BPT_F32 or BPT_BF16");
  if (d->dtype != BPT_BF16) return fail(BPT_ERR_UNSUPPORTED, "attention backward takes BPT_BF16 only");
  const int dh = d->d_model / d->n_heads;
  if (dh != 64 && dh != 128) return fail(BPT_ERR_UNSUPPORTED, "head size %d unsupported (64 or 128)", dh);
  const size_t np = round_up((size_t)d->seq_len, 128);
  if ((size_t)d->batch * np * (size_t)d->d_model >= ((size_t)1 << 31))
    return fail(BPT_ERR_SHAPE, "batch * seq_len * d_model exceeds the 31-bit element index range");
  if (d->window < 0 || d->chunk < 0) return fail(BPT_ERR_SHAPE, "window and chunk must be >= 0");
  if ((d->window || d->chunk) && !d->causal)
    return fail(BPT_ERR_SHAPE, "window and chunk apply to the causal mask only");
  if (d->window && d->chunk) return fail(BPT_ERR_SHAPE, "window and chunk cannot be combined");
  if (d->n_kv_heads < 0 || (d->n_kv_heads && d->n_heads % d->n_kv_heads != 0))
    return fail(BPT_ERR_SHAPE, "n_kv_heads %d must be 0 or divide n_heads %d", d->n_kv_heads,
                d->n_heads);
  return BPT_OK;
}

int attn_kv_heads(const bpt_attn_desc_t* d) { return d->n_kv_heads ? d->n_kv_heads : d->n_heads; }

// The two row statistics first, then the transposed copies, each on a 256-byte boundary.
size_t attn_bwd_layout(const bpt_attn_desc_t* d, size_t* stat_bytes, size_t* packed_bytes) {
  const size_t np = round_up((size_t)d->seq_len, 128);
  const size_t sb = round_up((size_t)d->batch * d->n_heads * np * sizeof(float), kAlign);
  const size_t pb = round_up((size_t)d->batch * np * d->d_model * 2, kAlign);
  if (stat_bytes) *stat_bytes = sb;
  if (packed_bytes) *packed_bytes = pb;
  return 2 * sb + (size_t)bpt::kAttnBwdPacked * pb;
}

}  // namespace

extern "C" {

size_t bpt_layer_workspace_bytes(const bpt_layer_desc_t* desc) {
  if (validate_desc(desc) != BPT_OK) return 0;
  if (is_empty(desc)) return 0;
  return layout(desc, false).total;
}

size_t bpt_stack_workspace_bytes(const bpt_layer_desc_t* desc, int32_t n_layers) {
  if (validate_desc(desc) != BPT_OK) return 0;
  if (n_layers < 1) {
    fail(BPT_ERR_SHAPE, "n_layers must be >= 1");
    return 0;
  }
  if (is_empty(desc)) return 0;
  return layout(desc, n_layers > 1 && desc->out_dtype != BPT_F32).total;
}

bpt_status_t bpt_layer_fwd(const bpt_layer_desc_t* desc, const void* X,
                           const bpt_layer_weights_t* weights, void* Z, void* workspace,
                           size_t workspace_bytes, void* hip_stream) {
  return bpt_layer_fwd_profiled(desc, X, weights, Z, workspace, workspace_bytes, hip_stream,
                                nullptr);
}

bpt_status_t bpt_layer_fwd_profiled(const bpt_layer_desc_t* desc, const void* X,
                                    const bpt_layer_weights_t* weights, void* Z, void* workspace,
                                    size_t workspace_bytes, void* hip_stream,
                                    void* const events[5]) {
  g_err[0] = 0;
  if (events)
    for (int i = 0; i < 5; ++i)
      if (!events[i]) return fail(BPT_ERR_NULL, "events[%d] is NULL", i);
  return layer_call(desc, X, weights, Z, nullptr, workspace, workspace_bytes, hip_stream, events);
}

bpt_status_t bpt_layer_fwd_lse(const bpt_layer_desc_t* desc, const void* X,
                               const bpt_layer_weights_t* weights, void* Z, float* lse,
                               void* workspace, size_t workspace_bytes, void* hip_stream) {
  g_err[0] = 0;
  bpt_status_t st = validate_desc(desc);
  if (st != BPT_OK) return st;
  if (is_empty(desc)) return BPT_OK;
  if (!lse) return fail(BPT_ERR_NULL, "lse is NULL");
  if (!aligned16(lse)) return fail(BPT_ERR_ALIGN, "lse is not 16-byte aligned");
  return layer_call(desc, X, weights, Z, lse, workspace, workspace_bytes, hip_stream, nullptr);
}

bpt_status_t bpt_stack_fwd(const bpt_layer_desc_t* desc, int32_t n_layers, const void* X,
                           const bpt_layer_weights_t* layers, void* Z, void* workspace,
                           size_t workspace_bytes, void* hip_stream) {
  g_err[0] = 0;
  bpt_status_t st = validate_desc(desc);
  if (st != BPT_OK) return st;
  if (n_layers < 1) return fail(BPT_ERR_SHAPE, "n_layers must be >= 1");
  if (is_empty(desc)) return BPT_OK;
  if (!layers) return fail(BPT_ERR_NULL, "layers is NULL");
  for (int i = 0; i < n_layers; ++i)
    if ((st = validate_weights(&layers[i], i)) != BPT_OK) return st;
  const bool resid = n_layers > 1 && desc->out_dtype != BPT_F32;
  const bpt::WorkspaceLayout L = layout(desc, resid);
  if ((st = validate_buffers(desc, X, Z, workspace, workspace_bytes, L.total)) != BPT_OK) return st;
  // The fp32 residual stream lives in Z itself when Z is fp32, else in the
  // workspace. Each epilogue tile reads its residual rows before writing the
  // same rows, so layers after the first update it in place.
  void* R = resid ? static_cast<char*>(workspace) + L.resid_off : Z;
  for (int i = 0; i < n_layers; ++i) {
    bpt::LayerLaunch p = make_launch(desc, L, workspace);
    const bool last = i == n_layers - 1;
    p.x = i == 0 ? X : R;
    p.x_f32 = i == 0 ? desc->dtype == BPT_F32 : 1;
    p.z = last ? Z : R;
    p.z_f32 = last ? desc->out_dtype == BPT_F32 : 1;
    p.w = layers[i];
    if ((st = run(p, hip_stream)) != BPT_OK) return st;
  }
  return BPT_OK;
}

bpt_status_t bpt_layer_fwd_noalloc(const bpt_layer_desc_t* desc, const void* X,
                                   const bpt_layer_weights_t* weights, void* Z, void* hip_stream) {
  g_err[0] = 0;
  bpt_status_t st = validate_desc(desc);
  if (st != BPT_OK) return st;
  if (is_empty(desc)) return BPT_OK;
  if ((st = validate_weights(weights, 0)) != BPT_OK) return st;
  const bpt::WorkspaceLayout L = layout(desc, false);
  if (L.total > bpt::kNoallocScratchBytes)
    return fail(BPT_ERR_WORKSPACE,
                "this layer needs %zu bytes of workspace; the fixed scratch of the no-allocation "
                "entry point holds %zu",
                L.total, bpt::kNoallocScratchBytes);
  // the caller's buffers first (no device access for these checks)
  if ((st = validate_buffers(desc, X, Z, nullptr, 0, 0)) != BPT_OK) return st;
  char msg[256] = "";
  void* ws = nullptr;
  if (bpt::noalloc_scratch(&ws, msg, sizeof(msg))) return fail(BPT_ERR_HIP, "%s", msg);
  if ((st = validate_buffers(desc, X, Z, ws, bpt::kNoallocScratchBytes, L.total)) != BPT_OK)
    return st;
  bpt::LayerLaunch p = make_launch(desc, L, ws);
  p.x = X;
  p.x_f32 = desc->dtype == BPT_F32;
  p.z = Z;
  p.z_f32 = desc->out_dtype == BPT_F32;
  p.w = *weights;
  return run(p, hip_stream);
}

size_t bpt_attention_bwd_workspace_bytes(const bpt_attn_desc_t* desc) {
  if (validate_attn_desc(desc) != BPT_OK) return 0;
  if (attn_empty(desc)) return 0;
  return attn_bwd_layout(desc, nullptr, nullptr);
}

bpt_status_t bpt_attention_bwd(const bpt_attn_desc_t* desc, const void* Q, const void* K,
                               const void* V, const void* O, const void* dO, const float* lse,
                               float* dQ, float* dK, float* dV, void* workspace,
                               size_t workspace_bytes, void* hip_stream) {
  return bpt_attention_bwd_profiled(desc, Q, K, V, O, dO, lse, dQ, dK, dV, workspace,
                                    workspace_bytes, hip_stream, nullptr);
}

bpt_status_t bpt_attention_bwd_profiled(const bpt_attn_desc_t* desc, const void* Q, const void* K,
                                        const void* V, const void* O, const void* dO,
                                        const float* lse, float* dQ, float* dK, float* dV,
                                        void* workspace, size_t workspace_bytes, void* hip_stream,
                                        void* const events[5]) {
  g_err[0] = 0;
  if (events)
    for (int i = 0; i < 5; ++i)
      if (!events[i]) return fail(BPT_ERR_NULL, "events[%d] is NULL", i);
  bpt_status_t st = validate_attn_desc(desc);
  if (st != BPT_OK) return st;
  if (attn_empty(desc)) return BPT_OK;
  const void* ptrs[] = {Q, K, V, O, dO, lse, dQ, dK, dV, workspace};
  const char* names[] = {"Q", "K", "V", "O", "dO", "lse", "dQ", "dK", "dV", "workspace"};
  for (int i = 0; i < 10; ++i) {
    if (!ptrs[i]) return fail(BPT_ERR_NULL, "%s is NULL", names[i]);
    if (!aligned16(ptrs[i])) return fail(BPT_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
  }
  size_t sbytes = 0, pbytes = 0;
  const size_t need = attn_bwd_layout(desc, &sbytes, &pbytes);
  if (workspace_bytes < need)
    return fail(BPT_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  const size_t rows = (size_t)desc->batch * desc->seq_len;
  const size_t dkv = (size_t)attn_kv_heads(desc) * (desc->d_model / desc->n_heads);
  const size_t in_b = rows * desc->d_model * 2, out_b = rows * desc->d_model * sizeof(float);
  const size_t kv_b = rows * dkv * 2, dkv_b = rows * dkv * sizeof(float);
  const size_t lse_b = rows * desc->n_heads * sizeof(float);
  // outputs and workspace against every other buffer
  const size_t sizes[] = {in_b, kv_b, kv_b, in_b, in_b, lse_b, out_b, dkv_b, dkv_b, need};
  for (int i = 6; i < 10; ++i)
    for (int j = 0; j < 10; ++j)
      if (j != i && overlap(ptrs[i], sizes[i], ptrs[j], sizes[j]))
        return fail(BPT_ERR_ALIAS, "%s overlaps %s", names[i], names[j]);
  bpt::AttnBwdLaunch p{};
  p.batch = desc->batch;
  p.seq_len = desc->seq_len;
  p.d_model = desc->d_model;
  p.n_heads = desc->n_heads;
  p.d_head = desc->d_model / desc->n_heads;
  p.causal = desc->causal;
  p.n_kv_heads = attn_kv_heads(desc);
  p.window = desc->window;
  p.chunk = desc->chunk;
  p.seq_pad = (int)round_up((size_t)desc->seq_len, 128);
  p.q = Q;
  p.k = K;
  p.v = V;
  p.out = O;
  p.dout = dO;
  p.lse = lse;
  p.dq = dQ;
  p.dk = dK;
  p.dv = dV;
  char* ws = static_cast<char*>(workspace);
  p.stat_d = reinterpret_cast<float*>(ws);
  p.stat_l2 = reinterpret_cast<float*>(ws + sbytes);
  for (int i = 0; i < bpt::kAttnBwdPacked; ++i) p.packed[i] = ws + 2 * sbytes + (size_t)i * pbytes;
  p.events = events;
  char msg[256] = "";
  if (bpt::launch_attention_bwd(p, hip_stream, msg, sizeof(msg))) return fail(BPT_ERR_HIP, "%s", msg);
  return BPT_OK;
}

size_t bpt_attention_fwd_workspace_bytes(const bpt_attn_desc_t* desc) {
  if (validate_attn_desc(desc) != BPT_OK) return 0;
  if (attn_empty(desc)) return 0;
  return 3 * round_up((size_t)desc->batch * round_up((size_t)desc->seq_len, 128) * desc->d_model * 2,
                      kAlign);
}

bpt_status_t bpt_attention_fwd(const bpt_attn_desc_t* desc, const void* Q, const void* K,
                               const void* V, void* O, float* lse, void* workspace,
                               size_t workspace_bytes, void* hip_stream) {
  g_err[0] = 0;
  bpt_status_t st = validate_attn_desc(desc);
  if (st != BPT_OK) return st;
  if (desc->window || desc->chunk || attn_kv_heads(desc) != desc->n_heads)
    return fail(BPT_ERR_UNSUPPORTED, "a ring step takes no window, chunk or grouped heads");
  if (attn_empty(desc)) return BPT_OK;
  const void* ptrs[] = {Q, K, V, O, lse, workspace};
  const char* names[] = {"Q", "K", "V", "O", "lse", "workspace"};
  for (int i = 0; i < 6; ++i) {
    if (!ptrs[i]) return fail(BPT_ERR_NULL, "%s is NULL", names[i]);
    if (!aligned16(ptrs[i])) return fail(BPT_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
  }
  const size_t need = bpt_attention_fwd_workspace_bytes(desc);
  if (workspace_bytes < need)
    return fail(BPT_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  const size_t rows = (size_t)desc->batch * desc->seq_len;
  const size_t in_b = rows * desc->d_model * 2, lse_b = rows * desc->n_heads * sizeof(float);
  const size_t sizes[] = {in_b, in_b, in_b, in_b, lse_b, need};
  for (int i = 3; i < 6; ++i)
    for (int j = 0; j < 6; ++j)
      if (j != i && overlap(ptrs[i], sizes[i], ptrs[j], sizes[j]))
        return fail(BPT_ERR_ALIAS, "%s overlaps %s", names[i], names[j]);
  bpt::AttnFwdLaunch p{};
  p.batch = desc->batch;
  p.seq_len = desc->seq_len;
  p.seq_pad = (int)round_up((size_t)desc->seq_len, 128);
  p.d_model = desc->d_model;
  p.n_heads = desc->n_heads;
  p.d_head = desc->d_model / desc->n_heads;
  p.causal = desc->causal;
  p.q = Q;
  p.k = K;
  p.v = V;
  p.o = O;
  p.lse = lse;
  const size_t pb = need / 3;
  for (int i = 0; i < 3; ++i) p.packed[i] = static_cast<char*>(workspace) + i * pb;
  char msg[256] = "";
  if (bpt::launch_attention_fwd(p, hip_stream, msg, sizeof(msg))) return fail(BPT_ERR_HIP, "%s", msg);
  return BPT_OK;
}

namespace {

// Shapes the ring entry points take: those of bpt_attention_fwd.
bpt_status_t validate_ring_desc(const bpt_attn_desc_t* d) {
  bpt_status_t st = validate_attn_desc(d);
  if (st != BPT_OK) return st;
  if (d->window || d->chunk || attn_kv_heads(d) != d->n_heads)
    return fail(BPT_ERR_UNSUPPORTED, "a ring share takes no window, chunk or grouped heads");
  return BPT_OK;
}

size_t ring_half_bytes(const bpt_attn_desc_t* d) {
  return round_up((size_t)d->batch * round_up((size_t)d->seq_len, 128) * d->d_model * 2, kAlign);
}

// Workspace of the share: Q in fragment layout, the fp32 running output in the
// same layout, the running statistic.
size_t ring_share_layout(const bpt_attn_desc_t* d, size_t* acc_off, size_t* lse_off) {
  const size_t q = ring_half_bytes(d);
  const size_t acc = 2 * q;
  const size_t lse = round_up((size_t)d->batch * d->n_heads * d->seq_len * 4, kAlign);
  if (acc_off) *acc_off = q;
  if (lse_off) *lse_off = q + acc;
  return q + acc + lse;
}

}  // namespace

size_t bpt_ring_kv_bytes(const bpt_attn_desc_t* desc) {
  if (validate_ring_desc(desc) != BPT_OK) return 0;
  if (attn_empty(desc)) return 0;
  return 2 * ring_half_bytes(desc);
}

bpt_status_t bpt_ring_pack_kv(const bpt_attn_desc_t* desc, const void* K, const void* V, void* kv,
                              size_t kv_bytes, void* hip_stream) {
  g_err[0] = 0;
  bpt_status_t st = validate_ring_desc(desc);
  if (st != BPT_OK) return st;
  if (attn_empty(desc)) return BPT_OK;
  const void* ptrs[] = {K, V, kv};
  const char* names[] = {"K", "V", "kv"};
  for (int i = 0; i < 3; ++i) {
    if (!ptrs[i]) return fail(BPT_ERR_NULL, "%s is NULL", names[i]);
    if (!aligned16(ptrs[i])) return fail(BPT_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
  }
  const size_t need = 2 * ring_half_bytes(desc);
  if (kv_bytes < need) return fail(BPT_ERR_WORKSPACE, "kv has %zu bytes, %zu needed", kv_bytes, need);
  const size_t in_b = (size_t)desc->batch * desc->seq_len * desc->d_model * 2;
  if (overlap(kv, need, K, in_b)) return fail(BPT_ERR_ALIAS, "kv overlaps K");
  if (overlap(kv, need, V, in_b)) return fail(BPT_ERR_ALIAS, "kv overlaps V");
  bpt::RingKvLaunch p{};
  p.batch = desc->batch;
  p.seq_len = desc->seq_len;
  p.seq_pad = (int)round_up((size_t)desc->seq_len, 128);
  p.d_model = desc->d_model;
  p.n_heads = desc->n_heads;
  p.d_head = desc->d_model / desc->n_heads;
  p.k = K;
  p.v = V;
  p.kv = kv;
  p.half_bytes = ring_half_bytes(desc);
  char msg[256] = "";
  if (bpt::launch_ring_pack_kv(p, hip_stream, msg, sizeof(msg))) return fail(BPT_ERR_HIP, "%s", msg);
  return BPT_OK;
}

size_t bpt_ring_share_workspace_bytes(const bpt_attn_desc_t* desc) {
  if (validate_ring_desc(desc) != BPT_OK) return 0;
  if (attn_empty(desc)) return 0;
  return ring_share_layout(desc, nullptr, nullptr);
}

bpt_status_t bpt_ring_share_fwd(const bpt_attn_desc_t* desc, int32_t n_shards, int32_t own,
                                const void* Q, const void* const* kv, void* O, float* lse,
                                void* workspace, size_t workspace_bytes, void* hip_stream) {
  g_err[0] = 0;
  bpt_status_t st = validate_ring_desc(desc);
  if (st != BPT_OK) return st;
  if (n_shards < 1 || n_shards > 4096) return fail(BPT_ERR_SHAPE, "n_shards %d must be in [1, 4096]", n_shards);
  if (own < 0 || own >= n_shards) return fail(BPT_ERR_SHAPE, "own %d must be in [0, n_shards)", own);
  if (attn_empty(desc)) return BPT_OK;
  if (!kv) return fail(BPT_ERR_NULL, "kv is NULL");
  // shards the share reads: all, or up to its own under the causal mask
  const int used = desc->causal ? own + 1 : n_shards;
  const size_t kv_b = 2 * ring_half_bytes(desc);
  size_t acc_off = 0, lse_off = 0;
  const size_t need = ring_share_layout(desc, &acc_off, &lse_off);
  const size_t rows = (size_t)desc->batch * desc->seq_len;
  const size_t in_b = rows * desc->d_model * 2, lse_b = rows * desc->n_heads * 4;
  const void* outs[] = {O, lse, workspace};
  const size_t out_b[] = {in_b, lse_b, need};
  const char* out_names[] = {"O", "lse", "workspace"};
  if (!Q) return fail(BPT_ERR_NULL, "Q is NULL");
  if (!aligned16(Q)) return fail(BPT_ERR_ALIGN, "Q is not 16-byte aligned");
  for (int i = 0; i < 3; ++i) {
    if (!outs[i]) return fail(BPT_ERR_NULL, "%s is NULL", out_names[i]);
    if (!aligned16(outs[i])) return fail(BPT_ERR_ALIGN, "%s is not 16-byte aligned", out_names[i]);
  }
  if (workspace_bytes < need)
    return fail(BPT_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  for (int s = 0; s < used; ++s) {
    if (!kv[s]) return fail(BPT_ERR_NULL, "kv[%d] is NULL", s);
    if (!aligned16(kv[s])) return fail(BPT_ERR_ALIGN, "kv[%d] is not 16-byte aligned", s);
  }
  for (int i = 0; i < 3; ++i) {
    if (overlap(outs[i], out_b[i], Q, in_b)) return fail(BPT_ERR_ALIAS, "%s overlaps Q", out_names[i]);
    for (int j = 0; j < 3; ++j)
      if (j != i && overlap(outs[i], out_b[i], outs[j], out_b[j]))
        return fail(BPT_ERR_ALIAS, "%s overlaps %s", out_names[i], out_names[j]);
    for (int s = 0; s < used; ++s)
      if (overlap(outs[i], out_b[i], kv[s], kv_b)) return fail(BPT_ERR_ALIAS, "%s overlaps kv[%d]", out_names[i], s);
  }
  bpt::RingShareLaunch p{};
  p.batch = desc->batch;
  p.seq_len = desc->seq_len;
  p.seq_pad = (int)round_up((size_t)desc->seq_len, 128);
  p.d_model = desc->d_model;
  p.n_heads = desc->n_heads;
  p.d_head = desc->d_model / desc->n_heads;
  p.causal = desc->causal;
  p.n_shards = n_shards;
  p.own = own;
  p.q = Q;
  p.kv = kv;
  p.kv_half_bytes = ring_half_bytes(desc);
  p.o = O;
  p.lse = lse;
  char* ws = static_cast<char*>(workspace);
  p.q_packed = ws;
  p.o_acc = reinterpret_cast<float*>(ws + acc_off);
  p.lse_acc = reinterpret_cast<float*>(ws + lse_off);
  char msg[256] = "";
  if (bpt::launch_ring_share(p, hip_stream, msg, sizeof(msg))) return fail(BPT_ERR_HIP, "%s", msg);
  return BPT_OK;
}

bpt_status_t bpt_attention_merge(const bpt_attn_desc_t* desc, float* O_acc, float* lse_acc,
                                 const void* O_part, const float* lse_part, void* hip_stream) {
  g_err[0] = 0;
  bpt_status_t st = validate_attn_desc(desc);
  if (st != BPT_OK) return st;
  if (attn_empty(desc)) return BPT_OK;
  const void* ptrs[] = {O_acc, lse_acc, O_part, lse_part};
  const char* names[] = {"O_acc", "lse_acc", "O_part", "lse_part"};
  for (int i = 0; i < 4; ++i) {
    if (!ptrs[i]) return fail(BPT_ERR_NULL, "%s is NULL", names[i]);
    if (!aligned16(ptrs[i])) return fail(BPT_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
  }
  const size_t rows = (size_t)desc->batch * desc->seq_len;
  const size_t sizes[] = {rows * desc->d_model * 4, rows * desc->n_heads * 4, rows * desc->d_model * 2,
                          rows * desc->n_heads * 4};
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 4; ++j)
      if (j != i && overlap(ptrs[i], sizes[i], ptrs[j], sizes[j]))
        return fail(BPT_ERR_ALIAS, "%s overlaps %s", names[i], names[j]);
  char msg[256] = "";
  if (bpt::launch_attention_merge(desc->batch, desc->seq_len, desc->n_heads,
                                  desc->d_model / desc->n_heads, O_acc, lse_acc, O_part, lse_part,
                                  hip_stream, msg, sizeof(msg)))
    return fail(BPT_ERR_HIP, "%s", msg);
  return BPT_OK;
}

namespace {

bpt_status_t validate_host_desc(const bpt_layer_desc_t* d, int32_t n_threads) {
  if (!d) return fail(BPT_ERR_NULL, "desc is NULL");
  if (d->batch < 0 || d->seq_len < 0) return fail(BPT_ERR_SHAPE, "batch and seq_len must be >= 0");
  if (d->d_model <= 0 || d->n_heads <= 0 || d->d_ff <= 0 || d->block_q <= 0)
    return fail(BPT_ERR_SHAPE, "d_model, n_heads, d_ff and block_q must be > 0");
  if (d->d_model % d->n_heads != 0)
    return fail(BPT_ERR_SHAPE, "d_model %d is not a multiple of n_heads %d", d->d_model, d->n_heads);
  if (d->causal != 0 && d->causal != 1) return fail(BPT_ERR_SHAPE, "causal must be 0 or 1");
  if (d->window < 0 || d->chunk < 0) return fail(BPT_ERR_SHAPE, "window and chunk must be >= 0");
  if ((d->window || d->chunk) && !d->causal)
    return fail(BPT_ERR_SHAPE, "window and chunk apply to the causal mask only");
  if (d->window && d->chunk) return fail(BPT_ERR_SHAPE, "window and chunk cannot be combined");
  if (d->n_kv_heads < 0 || (d->n_kv_heads && d->n_heads % d->n_kv_heads != 0))
    return fail(BPT_ERR_SHAPE, "n_kv_heads %d must be 0 or divide n_heads %d", d->n_kv_heads,
                d->n_heads);
  if (!(d->ln_eps > 0.0f) || !isfinite(d->ln_eps))
    return fail(BPT_ERR_SHAPE, "ln_eps must be finite and > 0");
  if ((d->dtype != BPT_F32 && d->dtype != BPT_BF16) ||
      (d->out_dtype != BPT_F32 && d->out_dtype != BPT_BF16))
    return fail(BPT_ERR_SHAPE, "dtype / out_dtype must be BPT_F32 or BPT_BF16");
  if (d->act != 0) return fail(BPT_ERR_UNSUPPORTED, "act %d unsupported (0 = GELU tanh)", d->act);
  if (d->precision != 0) return fail(BPT_ERR_UNSUPPORTED, "the host layer computes in fp32 (precision 0)");
  if (d->d_model % 8 || (d->d_model / d->n_heads) % 8 || d->d_ff % 8)
    return fail(BPT_ERR_UNSUPPORTED, "d_model, d_head and d_ff must be multiples of 8");
  if (n_threads < 1 || n_threads > 1024) return fail(BPT_ERR_SHAPE, "n_threads must be in [1, 1024]");
  if ((int64_t)d->batch * d->seq_len > (int64_t)INT32_MAX)
    return fail(BPT_ERR_SHAPE, "batch * seq_len exceeds the 32-bit row index range");
  return BPT_OK;
}

size_t host_workspace(const bpt_layer_desc_t* d, int32_t n_threads, size_t* kv_bytes) {
  const size_t kvb = round_up((size_t)d->batch * d->seq_len * kv_width(d) * sizeof(float), kAlign);
  if (kv_bytes) *kv_bytes = kvb;
  const size_t per = bpt::host_scratch_floats(d->d_model, d->n_heads, d->block_q) * sizeof(float);
  return 2 * kvb + (size_t)n_threads * round_up(per, kAlign);
}

}  // namespace

size_t bpt_layer_host_workspace_bytes(const bpt_layer_desc_t* desc, int32_t n_threads) {
  if (validate_host_desc(desc, n_threads) != BPT_OK) return 0;
  if (is_empty(desc)) return 0;
  return host_workspace(desc, n_threads, nullptr);
}

bpt_status_t bpt_layer_fwd_host(const bpt_layer_desc_t* desc, const void* X,
                                const bpt_layer_weights_t* weights, void* Z, void* workspace,
                                size_t workspace_bytes, int32_t n_threads) {
  g_err[0] = 0;
  bpt_status_t st = validate_host_desc(desc, n_threads);
  if (st != BPT_OK) return st;
  if (is_empty(desc)) return BPT_OK;
  if (!weights) return fail(BPT_ERR_NULL, "weights is NULL");
  const void* p[10] = {weights->ln1_g, weights->ln1_b, weights->w_q, weights->w_k, weights->w_v,
                       weights->w_o,   weights->ln2_g, weights->ln2_b, weights->w_1, weights->w_2};
  for (int i = 0; i < 10; ++i)
    if (!p[i]) return fail(BPT_ERR_NULL, "weights[0] entry %d is NULL", i);
  if (!X) return fail(BPT_ERR_NULL, "X is NULL");
  if (!Z) return fail(BPT_ERR_NULL, "Z is NULL");
  if (!workspace) return fail(BPT_ERR_NULL, "workspace is NULL");
  size_t kvb = 0;
  const size_t need = host_workspace(desc, n_threads, &kvb);
  if (workspace_bytes < need)
    return fail(BPT_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  if (((uintptr_t)workspace & 3u) != 0) return fail(BPT_ERR_ALIGN, "workspace is not 4-byte aligned");
  const size_t rows = (size_t)desc->batch * desc->seq_len;
  const size_t xb = rows * desc->d_model * esize(desc->dtype);
  const size_t zb = rows * desc->d_model * esize(desc->out_dtype);
  if (overlap(X, xb, Z, zb)) return fail(BPT_ERR_ALIAS, "X and Z overlap");
  if (overlap(workspace, need, X, xb)) return fail(BPT_ERR_ALIAS, "workspace overlaps X");
  if (overlap(workspace, need, Z, zb)) return fail(BPT_ERR_ALIAS, "workspace overlaps Z");
  bpt::HostLaunch L{};
  L.batch = desc->batch;
  L.seq_len = desc->seq_len;
  L.d_model = desc->d_model;
  L.n_heads = desc->n_heads;
  L.n_kv_heads = kv_heads(desc);
  L.d_kv = (int)kv_width(desc);
  L.d_ff = desc->d_ff;
  L.block_q = desc->block_q;
  L.causal = desc->causal;
  L.window = desc->window;
  L.chunk = desc->chunk;
  L.ln_eps = desc->ln_eps;
  L.x_f32 = desc->dtype == BPT_F32;
  L.w_f32 = desc->dtype == BPT_F32;
  L.z_f32 = desc->out_dtype == BPT_F32;
  L.x = X;
  L.w = *weights;
  L.z = Z;
  char* ws = static_cast<char*>(workspace);
  L.kbuf = reinterpret_cast<float*>(ws);
  L.vbuf = reinterpret_cast<float*>(ws + kvb);
  L.scratch = reinterpret_cast<float*>(ws + 2 * kvb);
  L.n_threads = n_threads;
  if (bpt::launch_layer_host(L)) return fail(BPT_ERR_UNSUPPORTED, "no host instance for these types");
  return BPT_OK;
}

namespace {

// The backward's limits on top of the forward's (bpt_layer_bwd).
bpt_status_t validate_bwd_desc(const bpt_layer_desc_t* d) {
  bpt_status_t st = validate_desc(d);
  if (st != BPT_OK) return st;
  if (d->dtype != BPT_BF16) return fail(BPT_ERR_UNSUPPORTED, "the layer backward takes BPT_BF16 only");
  if (d->precision != 0) return fail(BPT_ERR_UNSUPPORTED, "the layer backward computes at precision 0");
  if ((size_t)d->batch * seq_pad_of(d) * (size_t)d->d_model >= ((size_t)1 << 31))
    return fail(BPT_ERR_SHAPE, "batch * seq_len * d_model exceeds the 31-bit element index range");
  return BPT_OK;
}

// Byte offsets of the backward's workspace pieces. Buffers that are dead by the
// time a later one is written share its space: dA over dZ (bf16), [dQ dK dV] in
// bf16 ([rows, 3d]) over Q, K, V (one piece of 3 [rows, d]), dQ over Y and dLN1
// over dLN2 (fp32); of the transposed copies, dY^T over dZ^T, dQ^T over LN2(Y)^T
// and dK^T over A^T.
struct BwdLayout {
  size_t x1, q, k, v, attn, y2, dzb, dyb;   // bf16 [rows, d]
  size_t x1t, attnt, y2t, dzt, dvt;         // bf16 [d, rows_t]
  size_t y, dy2, dy, dk, dv;                // fp32 [rows, d]
  size_t stats1, stats2, lse_re, stat_d, stat_l2, packed[3];
  size_t ublk, hblk, dublk, dub, wt[4], partials, ln_part, total;
  int block_rows, blk_ld, rows_t, wgrad_splits, ffn_splits, ln_parts;
};

BwdLayout bwd_layout(const bpt_layer_desc_t* d) {
  BwdLayout L{};
  const size_t rows = (size_t)d->batch * d->seq_len, dm = d->d_model, f = d->d_ff;
  const size_t np = seq_pad_of(d), bh = (size_t)d->batch * d->n_heads;
  size_t r = (((size_t)1 << 26) / f) / 128 * 128;
  if (r < 128) r = 128;
  L.block_rows = (int)(r < rows ? r : rows);
  L.blk_ld = (int)round_up((size_t)L.block_rows, 8);
  L.rows_t = (int)round_up(rows, 8);
  // the product kernel's tiles are 256 x 256
  auto tiles_of = [](size_t m, size_t n) { return ((m + 255) / 256) * ((n + 255) / 256); };
  const size_t tiles = tiles_of(dm, dm);
  size_t splits = (512 + tiles - 1) / tiles;
  if (splits > 16) splits = 16;
  if (splits > rows / 256) splits = rows / 256;
  if (splits < 1) splits = 1;
  L.wgrad_splits = (int)splits;
  // dW_1, dW_2 per block: [d, d_ff] tiles, the block's rows split to reach ~256
  // workgroups (one per CU; more splits only add partial sums to write and add up),
  // each layer at least 1024 rows
  const size_t ftiles = tiles_of(dm, f) < tiles_of(f, dm) ? tiles_of(dm, f) : tiles_of(f, dm);
  size_t fsplits = (256 + ftiles - 1) / ftiles;
  if (fsplits > (size_t)L.block_rows / 1024) fsplits = (size_t)L.block_rows / 1024;
  if (fsplits > 16) fsplits = 16;
  if (fsplits < 1) fsplits = 1;
  L.ffn_splits = (int)fsplits;
  const size_t parts = (rows + 3) / 4;
  L.ln_parts = (int)(parts < 512 ? parts : 512);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += round_up(bytes, kAlign);
    return o;
  };
  const size_t rb = rows * dm * 2, rf = rows * dm * 4, tb = dm * (size_t)L.rows_t * 2;
  L.x1 = take(rb); L.q = take(3 * rb); L.k = L.q + rb; L.v = L.q + 2 * rb;
  L.attn = take(rb); L.y2 = take(rb); L.dzb = take(rb); L.dyb = take(rb);
  L.x1t = take(tb); L.attnt = take(tb); L.y2t = take(tb); L.dzt = take(tb); L.dvt = take(tb);
  L.y = take(rf); L.dy2 = take(rf); L.dy = take(rf); L.dk = take(rf); L.dv = take(rf);
  L.stats1 = take(rows * 8);
  L.stats2 = take(rows * 8);
  L.lse_re = take(bh * d->seq_len * 4);
  L.stat_d = take(bh * np * 4);
  L.stat_l2 = take(bh * np * 4);
  for (int i = 0; i < 3; ++i) L.packed[i] = take((size_t)d->batch * np * dm * 2);
  L.ublk = take(round_up(f, 256) * round_up((size_t)L.block_rows, 256) * 4);   // whole tiles, fragment order
  L.hblk = take(f * (size_t)L.blk_ld * 2);
  L.dublk = take(f * (size_t)L.blk_ld * 2);
  L.dub = take((size_t)L.block_rows * f * 2);
  L.wt[0] = take(dm * f * 2);   // W_1^T
  L.wt[1] = take(dm * f * 2);   // W_2^T
  L.wt[2] = take(dm * dm * 2);       // W_O^T
  L.wt[3] = take(3 * dm * dm * 2);   // W_Q^T | W_K^T | W_V^T
  const size_t pw = splits > 1 ? splits * dm * dm * 4 : 0, pf = fsplits > 1 ? fsplits * dm * f * 4 : 0;
  L.partials = take(pw > pf ? pw : pf);
  L.ln_part = take((size_t)L.ln_parts * 2 * dm * 4);
  L.total = off;
  return L;
}

}  // namespace

size_t bpt_layer_bwd_workspace_bytes(const bpt_layer_desc_t* desc) {
  if (validate_bwd_desc(desc) != BPT_OK) return 0;
  if (is_empty(desc)) return 0;
  return bwd_layout(desc).total;
}

bpt_status_t bpt_layer_bwd(const bpt_layer_desc_t* desc, const void* X,
                           const bpt_layer_weights_t* weights, const float* lse, const float* dZ,
                           float* dX, const bpt_layer_grads_t* grads, void* workspace,
                           size_t workspace_bytes, void* hip_stream) {
  g_err[0] = 0;
  bpt_status_t st = validate_bwd_desc(desc);
  if (st != BPT_OK) return st;
  if (is_empty(desc)) return BPT_OK;
  if ((st = validate_weights(weights, 0)) != BPT_OK) return st;
  if (!grads) return fail(BPT_ERR_NULL, "grads is NULL");
  const BwdLayout W = bwd_layout(desc);
  const size_t rows = (size_t)desc->batch * desc->seq_len, dm = desc->d_model, f = desc->d_ff;
  const size_t rd = rows * dm, dd = dm * dm, df = dm * f;
  const size_t kd = (size_t)kv_heads(desc) * (dm / desc->n_heads) * dm;   // W_K, W_V: [d_kv, d]
  // every buffer: the inputs, then the outputs (dX, the gradients, the workspace)
  const void* ptrs[24] = {X, weights->ln1_g, weights->ln1_b, weights->w_q, weights->w_k, weights->w_v,
                          weights->w_o, weights->ln2_g, weights->ln2_b, weights->w_1, weights->w_2, lse,
                          dZ, dX, grads->ln1_g, grads->ln1_b, grads->w_q, grads->w_k, grads->w_v,
                          grads->w_o, grads->ln2_g, grads->ln2_b, grads->w_1, grads->w_2};
  static const char* names[25] = {"X", "ln1_g", "ln1_b", "w_q", "w_k", "w_v", "w_o", "ln2_g", "ln2_b",
                                  "w_1", "w_2", "lse", "dZ", "dX", "grads.ln1_g", "grads.ln1_b",
                                  "grads.w_q", "grads.w_k", "grads.w_v", "grads.w_o", "grads.ln2_g",
                                  "grads.ln2_b", "grads.w_1", "grads.w_2", "workspace"};
  const size_t elems[24] = {rd, dm, dm, dd, kd, kd, dd, dm, dm, df, df,
                            (size_t)desc->batch * desc->n_heads * desc->seq_len, rd, rd,
                            dm, dm, dd, kd, kd, dd, dm, dm, df, df};
  const void* all[25];
  size_t bytes[25];
  for (int i = 0; i < 24; ++i) {
    all[i] = ptrs[i];
    bytes[i] = elems[i] * (i <= 10 ? 2 : 4);
  }
  all[24] = workspace;
  bytes[24] = W.total;
  for (int i = 11; i < 25; ++i) {
    if (!all[i]) return fail(BPT_ERR_NULL, "%s is NULL", names[i]);
    if (!aligned16(all[i])) return fail(BPT_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
  }
  if (!X) return fail(BPT_ERR_NULL, "X is NULL");
  if (!aligned16(X)) return fail(BPT_ERR_ALIGN, "X is not 16-byte aligned");
  if (workspace_bytes < W.total)
    return fail(BPT_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, W.total);
  for (int i = 13; i < 25; ++i)
    for (int j = 0; j < 25; ++j)
      if (j != i && overlap(all[i], bytes[i], all[j], bytes[j]))
        return fail(BPT_ERR_ALIAS, "%s overlaps %s", names[i], names[j]);
  char* ws = static_cast<char*>(workspace);
  auto F = [&](size_t o) { return reinterpret_cast<float*>(ws + o); };
  bpt::LayerBwdLaunch p{};
  p.batch = desc->batch;
  p.seq_len = desc->seq_len;
  p.seq_pad = (int)seq_pad_of(desc);
  p.d_model = desc->d_model;
  p.n_heads = desc->n_heads;
  p.d_ff = desc->d_ff;
  p.causal = desc->causal;
  p.n_kv_heads = kv_heads(desc);
  p.window = desc->window;
  p.chunk = desc->chunk;
  p.rows = (int)rows;
  p.rows_t = W.rows_t;
  p.ln_eps = desc->ln_eps;
  p.block_rows = W.block_rows;
  p.blk_ld = W.blk_ld;
  p.wgrad_splits = W.wgrad_splits;
  p.ffn_splits = W.ffn_splits;
  p.ln_parts = W.ln_parts;
  p.x = X;
  p.w = *weights;
  p.lse = lse;
  p.dz = dZ;
  p.dx = dX;
  p.g = *grads;
  p.x1 = ws + W.x1;
  p.q = ws + W.q;
  p.k = ws + W.k;
  p.v = ws + W.v;
  p.attn = ws + W.attn;
  p.y2 = ws + W.y2;
  p.dzb = ws + W.dzb;
  p.dyb = ws + W.dyb;
  p.da = ws + W.dzb;    // dZ (bf16) is dead once the FFN blocks are done
  p.dqkvb = ws + W.q;   // Q, K, V are dead once the attention backward is done
  p.x1t = ws + W.x1t;
  p.attnt = ws + W.attnt;
  p.y2t = ws + W.y2t;
  p.dzt = ws + W.dzt;
  p.dyt = ws + W.dzt;   // dZ^T is dead once the FFN blocks are done
  p.dqt = ws + W.y2t;   // LN2(Y)^T likewise
  p.dkt = ws + W.attnt; // A^T is dead once dW_O is formed, before the attention backward
  p.dvt = ws + W.dvt;
  p.hblk = ws + W.hblk;
  p.dublk = ws + W.dublk;
  p.dub = ws + W.dub;
  p.w1t = ws + W.wt[0];
  p.w2t = ws + W.wt[1];
  p.wot = ws + W.wt[2];
  p.wqkvt = ws + W.wt[3];
  p.ublk = F(W.ublk);
  p.y = F(W.y);
  p.dy2 = F(W.dy2);
  p.dy = F(W.dy);
  p.dq = F(W.y);        // Y is dead once the LN2 backward is done
  p.dk = F(W.dk);
  p.dv = F(W.dv);
  p.dx1 = F(W.dy2);     // dLN2 is dead once the LN2 backward is done
  p.stats1 = F(W.stats1);
  p.stats2 = F(W.stats2);
  p.lse_re = F(W.lse_re);
  p.stat_d = F(W.stat_d);
  p.stat_l2 = F(W.stat_l2);
  for (int i = 0; i < 3; ++i) p.packed[i] = ws + W.packed[i];
  p.partials = F(W.partials);
  p.ln_part = F(W.ln_part);
  char msg[256] = "";
  if (bpt::launch_layer_bwd(p, hip_stream, msg, sizeof(msg))) return fail(BPT_ERR_HIP, "%s", msg);
  return BPT_OK;
}

const char* bpt_status_str(bpt_status_t s) {
  switch (s) {
    case BPT_OK: return "ok";
    case BPT_ERR_NULL: return "null pointer";
    case BPT_ERR_SHAPE: return "invalid shape or option";
    case BPT_ERR_UNSUPPORTED: return "unsupported configuration";
    case BPT_ERR_ALIGN: return "misaligned pointer";
    case BPT_ERR_WORKSPACE: return "workspace too small";
    case BPT_ERR_ALIAS: return "overlapping buffers";
    case BPT_ERR_HIP: return "HIP launch failure";
  }
  return "unknown status";
}

const char* bpt_last_error(void) { return g_err; }

const char* bpt_version(void) { return "0.1.0"; }

}  // extern "C"
