"""FLOP, byte and activation-memory accounting of the BPT layer forward.

Formulas from "Blockwise Parallel Transformer — BPT" (aicassindra.com):
  * "FLOPs are unchanged": attention 4 N^2 d (QK^T and AV), QKVO projections
    8 N d^2, FFN (4d) 16 N d^2; attention dominates when N > 6d.
  * "Memory accounting" and the activation audit of "The bottleneck that survives
    FlashAttention": per layer 6 N d + 8 N d before fusion, 2 N d + O(b d) after.
  * "A worked example at 32k context": the BPT tile 8 b d.
  * "Choosing the block size": one block of b rows re-reads W_1 and W_2 (16 d^2
    bytes in bf16) for 16 b d^2 FLOPs, so the FFN's intensity is b FLOP per byte.
  * "On CPUs and small language models": the [N, 4d] hidden state versus a [b, 4d]
    tile.
"""
from __future__ import annotations


def visible_pairs(n: int, causal: bool, window: int = 0, chunk: int = 0) -> int:
    """(query, key) pairs one sequence's attention computes: N^2 without a mask,
    N (N + 1) / 2 causal; a window w leaves min(p + 1, w) keys to query p; chunked
    streaming with chunk C leaves min(N, (p // C + 1) C) keys to query p."""
    if not causal:
        return n * n
    if window:
        w = min(window, n)
        return w * (w + 1) // 2 + (n - w) * w
    if chunk:
        full, rest = divmod(n, chunk)
        # chunk c (0-based) holds C queries, each seeing (c + 1) C keys; the last,
        # partial chunk's queries see all n keys
        return chunk * chunk * full * (full + 1) // 2 + rest * n
    return n * (n + 1) // 2


def attention_flops(n: int, d: int, causal: bool, window: int = 0, chunk: int = 0) -> int:
    """Score and value products of one sequence: 2 matmuls x 2 FLOP per multiply-add
    over the visible (query, key) pairs: 4 N^2 d without a mask, 2 d N (N + 1)
    causal (visible_pairs for the window and chunk masks)."""
    return 4 * d * visible_pairs(n, causal, window, chunk)


def attention_bwd_flops(n: int, d: int, causal: bool) -> int:
    """Attention backward of one sequence: the scores recomputed from the saved
    statistics, then dV = P^T dO, dP = dO V^T, dQ = dS K and dK = dS^T Q, five
    products over the visible (query, key) pairs: 2.5 times attention_flops."""
    return 5 * attention_flops(n, d, causal) // 2


def projection_flops(n: int, d: int, d_kv: int | None = None) -> int:
    """W_Q, W_K, W_V, W_O: 4 matmuls of [N, d] x [d, d] (8 N d^2); with d_kv-wide
    key/value projections (grouped-query attention) W_K and W_V are [d, d_kv]."""
    d_kv = d if d_kv is None else d_kv
    return 4 * n * d * d + 4 * n * d * d_kv


def ffn_flops(n: int, d: int, d_ff: int) -> int:
    """W_1 [d, d_ff] and W_2 [d_ff, d]: 4 N d d_ff, i.e. 16 N d^2 at d_ff = 4d."""
    return 4 * n * d * d_ff


def layer_flops(n: int, d: int, d_ff: int, causal: bool, window: int = 0, chunk: int = 0,
                d_kv: int | None = None) -> int:
    """Algorithmic FLOPs of one layer on one sequence of N tokens."""
    return (attention_flops(n, d, causal, window, chunk) + projection_flops(n, d, d_kv)
            + ffn_flops(n, d, d_ff))


def layer_bwd_flops(n: int, d: int, d_ff: int, causal: bool) -> int:
    """Backward of one layer on one sequence, without recomputation: each dense
    product y = x W has two in the backward (dx = dy W^T and dW = x^T dy), twice the
    forward's projection and FFN FLOPs; the attention backward is attention_bwd_flops.
    (The block-recompute backward also runs the forward's products once more:
    layer_flops on top of this.)"""
    return 2 * (projection_flops(n, d) + ffn_flops(n, d, d_ff)) + attention_bwd_flops(n, d, causal)


def workload_flops(batch: int, n: int, d: int, d_ff: int, causal: bool, n_layers: int = 1,
                   window: int = 0, chunk: int = 0, d_kv: int | None = None) -> int:
    return batch * n_layers * layer_flops(n, d, d_ff, causal, window, chunk, d_kv)


def attention_crossover_tokens(d: int) -> int:
    """Smallest N where 4 N^2 d exceeds 8 N d^2 + 16 N d^2 (N > 6 d), at d_ff = 4d."""
    return 6 * d + 1


def activation_elems_after_flash(n: int, d: int) -> dict:
    """The per-layer activation audit once the h N^2 logits are gone (elements)."""
    return {"residual": n * d, "qkv": 3 * n * d, "attn_out_proj": 2 * n * d,
            "ffn_hidden": 8 * n * d, "rest": 6 * n * d}


def logits_elems(n: int, n_heads: int) -> int:
    return n_heads * n * n


def bpt_tile_elems(b: int, d: int) -> int:
    """The block-shaped live set the fused loop keeps for the FFN: two [b, 4d] tiles."""
    return 8 * b * d


def ffn_block_intensity(b: int) -> float:
    """FLOP per byte of W_1 + W_2 (bf16) re-read once per block of b rows."""
    d = 1  # cancels
    return (16 * b * d * d) / (16 * d * d)


def ffn_hidden_bytes(n: int, d_ff: int, bytes_per_elem: int = 2) -> int:
    """One [N, d_ff] hidden tensor."""
    return n * d_ff * bytes_per_elem


def ffn_tile_bytes(b: int, d_ff: int, bytes_per_elem: int = 2) -> int:
    """One [b, d_ff] hidden tile."""
    return b * d_ff * bytes_per_elem
