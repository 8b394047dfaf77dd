/*
 * bpt.h -- C ABI of the Blockwise Parallel Transformer (BPT) layer forward on
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed ("Blockwise Parallel Transformer — BPT", aicassindra.com,
 * section "The fused blockwise algorithm"): one pre-LN transformer layer,
 * Z = Y + FFN(LN2(Y)) with Y = X + Attention(LN1(X)) W_O, evaluated block by block.
 * Each block of b query rows attends to the key/value blocks one at a time,
 * keeping per row and head a running maximum of the scaled scores, the running
 * sum of their exponentials and the running exponential-weighted sum of values
 * (both rescaled when the maximum grows); the normalised result goes through W_O
 * and the residual, then LN2, W_1, GELU (tanh form) and W_2 and the second
 * residual finish those rows. The block's [b, d_ff] hidden state only ever
 * exists on chip (registers and LDS). Heads are contiguous d_k = d_model /
 * n_heads column slices, concatenated in order; scores are scaled by
 * 1/sqrt(d_k). Under the causal mask, key/value blocks that lie wholly after
 * the query block are never visited ("Pitfalls and misconceptions"). K and V
 * are projected once per layer rather than once per inner-loop visit (a
 * documented deviation from the page; the values are identical).
 *
 * Conventions shared by every entry point
 *  - Pointers named X, Z, workspace and every weight are DEVICE pointers to
 *    contiguous row-major arrays, 16-byte aligned. Descriptors are HOST pointers.
 *  - X: [batch * seq_len, d_model], sequences stacked row-wise, element type
 *    desc->dtype.  Z: same shape, element type desc->out_dtype.
 *  - LN parameters ln1_g, ln1_b, ln2_g, ln2_b: [d_model], type desc->dtype.
 *    LN is (x - mean) / sqrt(biased variance + ln_eps) * g + b over the feature axis.
 *  - Projection matrices are stored TRANSPOSED relative to the pages' y = x W
 *    notation, i.e. row-major [out, in] (the torch.nn.Linear layout):
 *      w_q, w_k, w_v, w_o: [d_model, d_model];  w_1: [d_ff, d_model];
 *      w_2: [d_model, d_ff].  No linear biases.
 *  - dtype BPT_F32: every product runs in fp32 (fp32 matrix cores).
 *    dtype BPT_BF16: products take bf16 operands with fp32 accumulation;
 *    softmax, LN, GELU and the residual stream are fp32.
 *  - The library never allocates device memory. All transient state lives in
 *    the caller's workspace, whose size the *_workspace_bytes functions return.
 *  - Asynchronous: a call only validates on the host and enqueues kernels on
 *    hip_stream (a hipStream_t; NULL = the default stream). Results are valid
 *    once the stream has been synchronised. Buffers must stay alive until then.
 *  - Errors: every argument is validated on the host before anything is
 *    enqueued; a non-zero status means nothing was enqueued, except
 *    BPT_ERR_HIP, returned when a launch fails (earlier launches of the same
 *    call may then have been enqueued). bpt_last_error() gives a
 *    human-readable detail for the calling thread. No C++ exception crosses
 *    this interface.
 *  - Thread-safe and reentrant: no mutable global state.
 */
#ifndef BPT_H_
#define BPT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { BPT_F32 = 0, BPT_BF16 = 1 } bpt_dtype_t;

typedef enum {
  BPT_OK = 0,
  BPT_ERR_NULL = 1,        /* a required pointer is NULL */
  BPT_ERR_SHAPE = 2,       /* a size is negative, or sizes disagree */
  BPT_ERR_UNSUPPORTED = 3, /* valid, but outside what the kernels implement */
  BPT_ERR_ALIGN = 4,       /* a device pointer is not 16-byte aligned */
  BPT_ERR_WORKSPACE = 5,   /* workspace smaller than *_workspace_bytes */
  BPT_ERR_ALIAS = 6,       /* X, Z or workspace overlap */
  BPT_ERR_HIP = 7          /* a HIP launch failed; see bpt_last_error() */
} bpt_status_t;

/* Shape and options of one layer (and of every layer of a stack). */
typedef struct {
  int32_t batch;      /* sequences; 0 gives an empty call that enqueues nothing  */
  int32_t seq_len;    /* tokens per sequence N; 0 likewise                      */
  int32_t d_model;    /* d; one of the sizes listed below                        */
  int32_t n_heads;    /* h; d_k = d_model / n_heads must be 64 or 128            */
  int32_t d_ff;       /* FFN width (4 d in the pages); a multiple of 256         */
  int32_t block_q;    /* b: query rows per outer-loop block; 64 or 128           */
  int32_t block_kv;   /* key/value rows per inner-loop block; 64 or 128          */
  int32_t causal;     /* 1: key j visible to query p iff j <= p; 0: no mask      */
  float ln_eps;       /* LN epsilon, > 0 (1e-5 is usual)                         */
  int32_t dtype;      /* bpt_dtype_t of X, the weights and the LN parameters     */
  int32_t out_dtype;  /* bpt_dtype_t of Z                                        */
  int32_t act;        /* 0 = GELU, tanh form (the only value)                    */
  int32_t precision;  /* 0: bf16 operands, fp32 accumulation; 1 (BPT_BF16 only):
                         every operand computed on the GPU (LN outputs, Q, K, V,
                         P, O, the FFN hidden state) is carried as a pair of bf16
                         values hi + lo (~16 significant bits), each product
                         taken over both halves; the FFN then runs staged (see
                         the workspace note)                                    */
  int32_t window;     /* 0: none. w > 0 (causal only): query p sees keys
                         max(0, p - w + 1) .. p ("transformer-cost" page, Section
                         5, the windowed mask)                                  */
  int32_t chunk;      /* 0: none. C > 0 (causal only, not with window): query p
                         sees every key j with j / C <= p / C, its whole chunk and
                         the earlier ones (same section, chunked streaming)     */
  int32_t n_kv_heads; /* key/value heads g (0: n_heads). Grouped-query attention
                         (same page, MQA and GQA): query head h reads key/value
                         head h / (n_heads / g); g must divide n_heads; 1 is MQA.
                         W_K and W_V are then [g * d_head, d_model]             */
} bpt_layer_desc_t;

/* Device pointers to one layer's parameters (layouts above; with n_kv_heads = g,
 * w_k and w_v are [g * d_head, d_model]). */
typedef struct {
  const void *ln1_g, *ln1_b, *w_q, *w_k, *w_v, *w_o;
  const void *ln2_g, *ln2_b, *w_1, *w_2;
} bpt_layer_weights_t;

/* Kernel instances exist for d_model 256, 512, 768, 1024, 2048, 4096 (BPT_BF16)
 * and 128, 256 (BPT_F32), head sizes 64 and 128, block_q and block_kv 64 or 128
 * (BPT_F32 with head size 128: block_kv 64), d_ff a multiple of 256. Any other
 * combination returns BPT_ERR_UNSUPPORTED before anything is enqueued, and so
 * does a shape whose matrix-product operands reach 4 GiB (e.g. 8 x 131072 tokens
 * at d_model 2048). Batch and sequence length are free otherwise; a sequence
 * length that is not a multiple of the block sizes gets a shorter last block.
 * The FFN epilogue: d_model up to 1024 in bf16 (or fp32) finishes each row tile
 * on one compute unit; d_model 2048 and 4096 (bf16, or bf16 pairs) finish tiles
 * of 128 rows on clusters of d_model / 512 compute units that exchange the LN2
 * operand and chunks of 256 d_model / 512 hidden units (d_ff must be a multiple
 * of that chunk); other shapes (bf16 pairs up to d_model 1024, or a d_ff that is
 * not such a multiple) run the FFN over blocks of rows, one GEMM at a time. */

/* Bytes of workspace bpt_layer_fwd needs for *desc (0 for an empty call), or 0
 * with bpt_last_error() set when desc is invalid ("Blockwise Parallel Transformer
 * — BPT", section "Memory accounting: what actually shrinks": per layer only the
 * residual-stream-shaped tensors and block-shaped tiles remain). Holds, in the
 * compute type: LN1(X) [rows rounded up to 256, d_model]; Q (reused for the
 * attention output), K and V^T, each [rows, d_model]; and a copy of the six
 * projection matrices repacked in matrix-core fragment order (4 d_model^2 +
 * 2 d_model d_ff elements). Nothing of size rows x d_ff or seq_len x seq_len is
 * ever part of it. d_model 2048 and 4096 add the clusters' exchange regions,
 * whose size does not depend on the rows: (256 / G) regions, G = d_model / 512,
 * each holding LN2 of a 128-row tile [128, d_model], two hidden chunks [128,
 * 256 G] and per-row statistics (about 64 MiB in all, twice that in bf16 pairs),
 * plus 4 KiB of counters. The row-block FFN (see above) instead adds one block of
 * the hidden state, [h, d_ff] with h = 2^25 / d_model rounded down to a multiple
 * of 256, at least 4096 and at most rows rounded up to 256, and keeps Y fp32
 * [rows, d_model] over the K and V^T space. precision 1 doubles every activation
 * buffer (the lo halves). */
size_t bpt_layer_workspace_bytes(const bpt_layer_desc_t* desc);
/* With g = n_kv_heads key/value heads, K and V^T are [rows, g * d_head] and the
 * packed projection block is [d_model + 2 kvp, d_model] with kvp = g * d_head
 * rounded up to 256 (the K and V parts are padded to whole product tiles); on the
 * row-block FFN the K and V^T space is at least the fp32 Y [rows, d_model]. */

/* Workspace of bpt_stack_fwd (same section): the layer workspace, reused by
 * every layer, plus one fp32 residual buffer [rows, d_model] when n_layers > 1
 * and out_dtype is not BPT_F32. */
size_t bpt_stack_workspace_bytes(const bpt_layer_desc_t* desc, int32_t n_layers);

/* One layer: Z = layer(X). X and Z must not overlap; workspace must overlap
 * neither. workspace_bytes >= bpt_layer_workspace_bytes(desc). */
bpt_status_t bpt_layer_fwd(const bpt_layer_desc_t* desc, const void* X,
                           const bpt_layer_weights_t* weights, void* Z,
                           void* workspace, size_t workspace_bytes, void* hip_stream);

/* bpt_layer_fwd that also records five caller-created hipEvent_t handles
 * (events: a HOST array of 5) on hip_stream, for timing each kernel:
 * events[0] before the LN1 statistics, [1] after them, [2] after the QKV
 * projection, [3] after attention, [4] after the FFN epilogue. The computation
 * and every other rule are those of bpt_layer_fwd; events may be NULL (then it
 * is bpt_layer_fwd), but not a NULL entry (BPT_ERR_NULL). */
bpt_status_t bpt_layer_fwd_profiled(const bpt_layer_desc_t* desc, const void* X,
                                    const bpt_layer_weights_t* weights, void* Z,
                                    void* workspace, size_t workspace_bytes, void* hip_stream,
                                    void* const events[5]);

/* bpt_layer_fwd that also writes the attention statistic the backward pass
 * needs. "Blockwise Parallel Transformer — BPT" (aicassindra.com), section "The
 * backward pass": the forward keeps only each row's softmax statistics (m, l),
 * from which every block's softmax is recomputed exactly; the FlashAttention
 * paragraph of the transformer-cost page (raminaeye.github.io) likewise. A
 * running maximum m and its sum l are not unique (any later maximum rescales
 * both); the number they fix, m + ln l, is:
 *   lse[(b * n_heads + h) * seq_len + p] = ln sum_{j visible to p} exp(q_p . k_j / sqrt(d_head))
 * for sequence b, head h, query position p (fp32, DEVICE pointer, batch *
 * n_heads * seq_len floats, 16-byte aligned, overlapping neither X, Z nor the
 * workspace: BPT_ERR_NULL, BPT_ERR_ALIGN, BPT_ERR_ALIAS). Written by the same
 * asynchronous launches as Z; every other argument and rule is bpt_layer_fwd's. */
bpt_status_t bpt_layer_fwd_lse(const bpt_layer_desc_t* desc, const void* X,
                               const bpt_layer_weights_t* weights, void* Z, float* lse,
                               void* workspace, size_t workspace_bytes, void* hip_stream);

/* Shape of one multi-head attention (the attention step of a layer). */
typedef struct {
  int32_t batch;      /* sequences; 0 gives an empty call that enqueues nothing  */
  int32_t seq_len;    /* tokens per sequence N; 0 likewise                      */
  int32_t d_model;    /* n_heads * d_head                                        */
  int32_t n_heads;    /* d_head = d_model / n_heads: 64 or 128                   */
  int32_t causal;     /* 1: key j visible to query p iff j <= p; 0: no mask      */
  int32_t dtype;      /* of Q, K, V, O and dO: BPT_BF16 (the only value)         */
  int32_t window;     /* as bpt_layer_desc_t (causal only; bpt_attention_bwd)     */
  int32_t chunk;      /* as bpt_layer_desc_t (causal only; bpt_attention_bwd)     */
  int32_t n_kv_heads; /* as bpt_layer_desc_t (bpt_attention_bwd): K, V, dK and dV
                         are then [batch * seq_len, n_kv_heads * d_head]        */
} bpt_attn_desc_t;

/* (bpt_attention_fwd and bpt_attention_merge take window = chunk = 0 and
 * n_kv_heads 0 or n_heads.)
 * Bytes of workspace bpt_attention_bwd needs (0 for an empty call, or 0 with
 * bpt_last_error() set when desc is invalid): two fp32 row statistics [batch,
 * n_heads, Np] (-D, D = rowsum(dO * O), and lse in base 2), with Np = seq_len rounded
 * up to 128, and transposed bf16 copies of K, Q and dO, each [batch * Np,
 * d_model]. Nothing of size seq_len x seq_len. */
size_t bpt_attention_bwd_workspace_bytes(const bpt_attn_desc_t* desc);

/* Attention backward of one multi-head attention A = softmax(Q K^T / sqrt(d_head)) V
 * per sequence and head (masked as desc->causal says), from the saved row
 * statistics. "Blockwise Parallel Transformer — BPT" (aicassindra.com), section
 * "The backward pass": the forward keeps only each row's softmax statistics, and
 * each block's softmax is recomputed from them while the gradients accumulate;
 * the FlashAttention paragraph of the transformer-cost page (raminaeye.github.io)
 * likewise. With P = exp(Q_h K_h^T / sqrt(d_head) - lse) (the exact softmax) and
 * D = rowsum(dO_h * O_h):
 *   dV_h = P^T dO_h,  dS = P * (dO_h V_h^T - D),
 *   dQ_h = dS K_h / sqrt(d_head),  dK_h = dS^T Q_h / sqrt(d_head).
 *  - Q, K, V, O, dO: DEVICE pointers, bf16 [batch * seq_len, d_model] row-major,
 *    heads concatenated along the features as in the layer (O is the attention
 *    output A of the forward, dO the gradient of the loss with respect to it).
 *  - lse: DEVICE, fp32 [batch, n_heads, seq_len], the statistic
 *    bpt_layer_fwd_lse writes: lse = ln sum over visible keys of exp(score).
 *  - dQ, dK, dV: DEVICE, fp32 [batch * seq_len, d_model], written (not added to).
 *  - Every device pointer 16-byte aligned (BPT_ERR_ALIGN), none NULL
 *    (BPT_ERR_NULL); the outputs and the workspace overlap no other buffer
 *    (BPT_ERR_ALIAS); the inputs may overlap each other.
 *  - Asynchronous on hip_stream, errors as for every entry point. */
bpt_status_t bpt_attention_bwd(const bpt_attn_desc_t* desc, const void* Q, const void* K,
                               const void* V, const void* O, const void* dO, const float* lse,
                               float* dQ, float* dK, float* dV, void* workspace,
                               size_t workspace_bytes, void* hip_stream);

/* bpt_attention_bwd that also records five caller-created hipEvent_t handles
 * (events: a HOST array of 5) on hip_stream, for timing each kernel: events[0]
 * before the row statistics, [1] after them, [2] after the transposed copies,
 * [3] after the dQ kernel, [4] after the dK / dV kernel. events may be NULL (then
 * it is bpt_attention_bwd), but not a NULL entry (BPT_ERR_NULL). */
bpt_status_t bpt_attention_bwd_profiled(const bpt_attn_desc_t* desc, const void* Q, const void* K,
                                        const void* V, const void* O, const void* dO,
                                        const float* lse, float* dQ, float* dK, float* dV,
                                        void* workspace, size_t workspace_bytes, void* hip_stream,
                                        void* const events[5]);

/* The same layer on the host CPU: the fused blockwise loop of the BPT page (and
 * its section "On CPUs and small language models": per block of block_q rows the
 * [block_q, d_ff] hidden state is produced and consumed in cache-sized chunks and
 * never written out), query blocks spread over n_threads threads (>= 1). X, Z,
 * the weights and the workspace are HOST pointers (no alignment needed); the
 * arithmetic is fp32 whatever dtype says (bf16 inputs are widened; a bf16 Z is
 * rounded to nearest even). Every descriptor field means what it means for
 * bpt_layer_fwd, with these limits instead of the GPU's kernel table: d_model,
 * d_head and d_ff multiples of 8, any block_q >= 1, precision 0, dtype BPT_F32
 * with fp32 or bf16 weights not distinguished (the weights have dtype's type).
 * Synchronous: returns when Z is written. The workspace holds K and V in fp32
 * [batch * seq_len, n_kv_heads * d_head] and per-thread block scratch. */
size_t bpt_layer_host_workspace_bytes(const bpt_layer_desc_t* desc, int32_t n_threads);
bpt_status_t bpt_layer_fwd_host(const bpt_layer_desc_t* desc, const void* X,
                                const bpt_layer_weights_t* weights, void* Z, void* workspace,
                                size_t workspace_bytes, int32_t n_threads);

/* One device's share of Ring Attention ("Blockwise Parallel Transformer — BPT",
 * section "BPT and Ring Attention": each device keeps its query shard while the
 * key/value shards travel around a ring). A step is the attention of the local
 * query shard against one arrived key/value shard of the same length N:
 * desc->causal = 1 for the device's own shard, 0 for an earlier one (a later one
 * is skipped). bpt_attention_fwd writes that step's normalised output O (bf16,
 * [batch * N, d_model] row-major, heads concatenated) and its statistic lse
 * ([batch, n_heads, N] fp32, as bpt_layer_fwd_lse); Q, K, V are bf16 row-major
 * DEVICE buffers like bpt_attention_bwd's. bpt_attention_merge folds one step into
 * the running state (O_acc fp32 [batch * N, d_model], lse_acc [batch, n_heads, N],
 * which start at 0 and -inf): lse = ln(e^lse_acc + e^lse_part), O_acc =
 * e^(lse_acc - lse) O_acc + e^(lse_part - lse) O_part; after every shard it holds
 * the attention of the query shard over the whole sequence. Errors and
 * asynchrony as for every entry point; the workspace holds packed copies of Q, K
 * and V ([batch * Np, d_model] bf16 each, Np = N rounded up to 128). */
size_t bpt_attention_fwd_workspace_bytes(const bpt_attn_desc_t* desc);
bpt_status_t bpt_attention_fwd(const bpt_attn_desc_t* desc, const void* Q, const void* K,
                               const void* V, void* O, float* lse, void* workspace,
                               size_t workspace_bytes, void* hip_stream);
bpt_status_t bpt_attention_merge(const bpt_attn_desc_t* desc, float* O_acc, float* lse_acc,
                                 const void* O_part, const float* lse_part, void* hip_stream);

/* One device's share of Ring Attention with the shards kept in the attention
 * kernels' layout ("Blockwise Parallel Transformer — BPT", aicassindra.com,
 * section "BPT and Ring Attention": each device keeps its query shard while the
 * key/value shards travel around the ring; each arrived shard is one more block
 * source for the inner loop). A device packs its own key/value shard once
 * (bpt_ring_pack_kv) and the packed shard is what travels; the share then runs its
 * query shard against every arrived shard and merges the steps' results inside
 * the attention kernel, as each row finishes, through the saved statistic
 * (lse = ln(e^a + e^b), O = e^(a - lse) O_a + e^(b - lse) O_b): no per-step copies
 * of Q, O or K/V and no separate merge pass.
 *  - desc: one shard's shape (batch sequences of seq_len tokens each), dtype
 *    BPT_BF16, window = chunk = 0, n_kv_heads 0 or n_heads.
 *  - bpt_ring_kv_bytes: bytes of a packed shard (K then V^T, each [batch * Np,
 *    d_model] bf16, Np = seq_len rounded up to 128); 0 (bpt_last_error set) when
 *    desc is invalid or an empty call.
 *  - bpt_ring_pack_kv: K, V DEVICE bf16 [batch * seq_len, d_model] row-major ->
 *    kv (DEVICE, kv_bytes >= bpt_ring_kv_bytes, overlapping neither K nor V).
 *  - bpt_ring_share_fwd: Q DEVICE bf16 [batch * seq_len, d_model]; kv a HOST
 *    array of n_shards (1..4096) DEVICE pointers to packed shards, shard s holding
 *    the tokens [s seq_len, (s + 1) seq_len) of the whole sequence and own the
 *    index of Q's shard. With desc->causal = 1, shards s < own are seen whole,
 *    shard own with the causal mask and shards s > own not at all (their pointers
 *    may be NULL); with causal = 0 every shard is seen whole. Writes O (DEVICE
 *    bf16 [batch * seq_len, d_model]) and lse (DEVICE fp32 [batch, n_heads,
 *    seq_len], the natural-log statistic over every key the rows saw). Workspace:
 *    bpt_ring_share_workspace_bytes (Q packed, an fp32 running output [batch * Np,
 *    d_model] and the running statistic). O, lse and the workspace overlap no
 *    other buffer; pointers 16-byte aligned; asynchronous on hip_stream. */
size_t bpt_ring_kv_bytes(const bpt_attn_desc_t* desc);
bpt_status_t bpt_ring_pack_kv(const bpt_attn_desc_t* desc, const void* K, const void* V, void* kv,
                              size_t kv_bytes, void* hip_stream);
size_t bpt_ring_share_workspace_bytes(const bpt_attn_desc_t* desc);
bpt_status_t bpt_ring_share_fwd(const bpt_attn_desc_t* desc, int32_t n_shards, int32_t own,
                                const void* Q, const void* const* kv, void* O, float* lse,
                                void* workspace, size_t workspace_bytes, void* hip_stream);

/* bpt_layer_fwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. The
 * workspace is not passed in: the library carves it from a fixed device array of
 * BPT_NOALLOC_SCRATCH_BYTES bytes that each GPU it runs on holds from the first
 * call until the process ends; the call itself allocates nothing (no hipMalloc,
 * no allocating library routine). X, Z and the weights are the caller's, with
 * every rule of bpt_layer_fwd. A descriptor whose bpt_layer_workspace_bytes
 * exceeds BPT_NOALLOC_SCRATCH_BYTES returns BPT_ERR_WORKSPACE before anything is
 * enqueued or any device is touched. Every call on one GPU shares that GPU's
 * array (it keeps the last call's contents; the layer overwrites all of it that
 * it reads), so calls that overlap on one GPU race: issue them on one stream,
 * or otherwise one after another. */
#define BPT_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
bpt_status_t bpt_layer_fwd_noalloc(const bpt_layer_desc_t* desc, const void* X,
                                   const bpt_layer_weights_t* weights, void* Z, void* hip_stream);

/* n_layers >= 1 layers applied in turn ("Blockwise Parallel Transformer — BPT",
 * section "A worked example at 32k context": a model is a stack of such layers
 * joined by the residual stream, and only that stream is sequence-shaped between
 * them), all with the shape of *desc; layers is a HOST array of n_layers weight
 * sets (each holding device pointers). Layer 0 reads X in desc->dtype; the
 * residual stream between layers is fp32; the last layer writes Z in
 * desc->out_dtype. No final LN. */
bpt_status_t bpt_stack_fwd(const bpt_layer_desc_t* desc, int32_t n_layers, const void* X,
                           const bpt_layer_weights_t* layers, void* Z,
                           void* workspace, size_t workspace_bytes, void* hip_stream);

/* Gradients of one layer's parameters: DEVICE pointers, fp32, each with the shape
 * and layout of the weight it belongs to (w_q, w_k, w_v, w_o [d_model, d_model],
 * w_1 [d_ff, d_model], w_2 [d_model, d_ff], all [out, in] row-major; the LN gains
 * and biases [d_model]). */
typedef struct {
  float *ln1_g, *ln1_b, *w_q, *w_k, *w_v, *w_o;
  float *ln2_g, *ln2_b, *w_1, *w_2;
} bpt_layer_grads_t;

/* Bytes of workspace bpt_layer_bwd needs for *desc (0 for an empty call), or 0
 * with bpt_last_error() set when desc is invalid or outside the backward's limits
 * (see bpt_layer_bwd). With rows = batch * seq_len and Np = seq_len rounded up to
 * 128, it holds: bf16 [rows, d_model] copies of LN1(X), Q, K, V, the attention
 * output A, LN2(Y), dZ, dY (dA, dQ, dK, dV over those that are dead by then);
 * bf16 transposed copies [d_model, rows] of LN1(X), A, LN2(Y), dZ and dV (dY, dQ,
 * dK over dead ones); fp32 [rows, d_model] Y (then dQ), dLN2 (then dLN1), dY, dK,
 * dV; per-row LN statistics; the attention operands in fragment order (3 x
 * [batch * Np, d_model] bf16) and its row statistics; one FFN block of r = min(rows,
 * 2^26 / d_ff) rows: U fp32 (rounded up to 256 x 256 tiles), H, dU (twice) bf16, each
 * [r, d_ff]; the six weights transposed in bf16; split-k partial sums (up to 16 x
 * [d_model, d_model] or a few [d_model, d_ff] fp32) and the LN column partials. The only d_ff-wide buffers are the block's: nothing of
 * size rows x d_ff or seq_len x seq_len. */
size_t bpt_layer_bwd_workspace_bytes(const bpt_layer_desc_t* desc);

/* Backward of one layer (bpt_layer_fwd's computation) by block recomputation.
 * "Blockwise Parallel Transformer — BPT" (aicassindra.com), section "The backward
 * pass": the forward keeps the layer input and each attention row's softmax
 * statistic; the backward recomputes what it needs from them (LN1(X), Q, K, V,
 * the attention output, Y and LN2(Y) here; each block's softmax inside the
 * attention backward; the FFN hidden state one block of rows at a time) while
 * the gradients of the weights accumulate. Given dZ = dL/dZ for a loss L:
 *  - dX = dL/dX (fp32 [rows, d_model], written);
 *  - grads: every parameter's gradient (bpt_layer_grads_t, written, not added to).
 * Arguments:
 *  - X, weights: the forward's input and parameters (DEVICE, bf16, layouts of
 *    bpt_layer_fwd).
 *  - lse: DEVICE fp32 [batch, n_heads, seq_len], the statistic bpt_layer_fwd_lse
 *    wrote for this X and these weights.
 *  - dZ: DEVICE fp32 [rows, d_model].
 * The masks (causal, window, chunk) and key/value heads (n_kv_heads; W_K, W_V and
 * their gradients [n_kv_heads * d_head, d_model]) are those of bpt_layer_fwd; a
 * key/value head's gradients sum over the query heads that read it.
 * Limits (else BPT_ERR_UNSUPPORTED before anything is enqueued): dtype BPT_BF16,
 * precision 0; every other shape bpt_layer_fwd takes (block_q, block_kv and
 * out_dtype do not matter here).
 * Products take bf16 operands (activations and gradients rounded to bf16 where
 * they enter a product) with fp32 accumulation; the weight gradients sum over the
 * rows in a fixed order, so repeated calls give identical bits. Every device
 * pointer 16-byte aligned (BPT_ERR_ALIGN), none NULL (BPT_ERR_NULL); dX, the
 * gradients and the workspace overlap no other buffer (BPT_ERR_ALIAS).
 * Asynchronous on hip_stream. */
bpt_status_t bpt_layer_bwd(const bpt_layer_desc_t* desc, const void* X,
                           const bpt_layer_weights_t* weights, const float* lse, const float* dZ,
                           float* dX, const bpt_layer_grads_t* grads, void* workspace,
                           size_t workspace_bytes, void* hip_stream);

/* Static text for a status code. */
const char* bpt_status_str(bpt_status_t status);

/* Detail of the calling thread's last non-OK status ("" if none). */
const char* bpt_last_error(void);

/* Library version, e.g. "0.1.0". */
const char* bpt_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BPT_H_ */
