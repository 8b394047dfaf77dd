"""The FLOP and memory accounting against the numbers the pages print."""
import json
import os

import pytest

from blockwise_attn_ffn_amd import accounting as A

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))


def test_worked_example_32k():
    g = G["worked_example_32k"]
    n, d, h, bpe, b = g["N"], g["d"], g["heads"], g["bytes_per_elem"], g["block"]
    audit = A.activation_elems_after_flash(n, d)
    assert round(audit["residual"] / 1e6, 1) == g["Nd_million_elems"]
    assert round(audit["residual"] * bpe / 1e6) == g["Nd_MB"]
    assert round(audit["ffn_hidden"] * bpe / 1e6) == g["ffn_hidden_8Nd_MB"]
    assert round(A.logits_elems(n, h) * bpe / 1e9, 1) == g["logits_hNN_GB"]
    assert round(A.bpt_tile_elems(b, d) / 1e6, 1) == g["bpt_tile_8bd_million_elems"]
    assert round(A.bpt_tile_elems(b, d) * bpe / 1e6, 1) == g["bpt_tile_8bd_MB"]
    assert audit["ffn_hidden"] // A.bpt_tile_elems(b, d) == g["reduction_N_over_b"] == n // b
    # the page's 32-layer line: 68.7 GB of FFN activations becomes 1.1 GB
    assert round(g["layers"] * audit["ffn_hidden"] * bpe / 1e9, 1) == g["ffn_activations_32_layers_GB_before"]
    assert round(g["layers"] * A.bpt_tile_elems(b, d) * bpe / 1e9, 1) == g["ffn_activations_32_layers_GB_after"]


def test_audit_totals():
    n, d = 1000, 64
    a = A.activation_elems_after_flash(n, d)
    assert a["rest"] == a["residual"] + a["qkv"] + a["attn_out_proj"] == 6 * n * d
    assert a["ffn_hidden"] == 8 * n * d


def test_flop_identity_and_crossover():
    g = G["crossover"]
    d = g["d"]
    n = 4096
    assert A.layer_flops(n, d, 4 * d, causal=False) == 4 * n * n * d + 8 * n * d * d + 16 * n * d * d
    c = A.attention_crossover_tokens(d)
    assert c == 6 * d + 1 == 24577
    assert abs(c - g["crossover_tokens_approx"]) / g["crossover_tokens_approx"] < 0.03
    assert A.attention_flops(c, d, False) > A.projection_flops(c, d) + A.ffn_flops(c, d, 4 * d)
    assert A.attention_flops(c - 1, d, False) == A.projection_flops(c - 1, d) + A.ffn_flops(c - 1, d, 4 * d)


def test_causal_flops_count_visible_pairs():
    # the causal count is exactly the number of (query, key) pairs with key <= query
    for n in (1, 2, 7, 128):
        pairs = sum(i + 1 for i in range(n))
        assert A.attention_flops(n, 64, True) == 4 * 64 * pairs


def test_slm_cpu_example():
    g = G["slm_cpu_example"]
    assert g["hidden_cols"] == 4 * g["d"]
    assert round(A.ffn_hidden_bytes(g["tokens"], g["hidden_cols"]) / 1e6) == g["hidden_MB_bf16"]
    assert round(A.ffn_tile_bytes(g["block"], g["hidden_cols"]) / 1e6) == g["tile_MB"]


@pytest.mark.parametrize("b", [64, 128, 512])
def test_block_intensity_is_block_size(b):
    assert A.ffn_block_intensity(b) == b


def test_workload_flops_of_the_five_workloads():
    # 0.134 GFLOP, 283.5 GFLOP, 1.787 TFLOP, 83.56 TFLOP, 87.96 TFLOP
    assert round(A.workload_flops(1, 256, 128, 512, False) / 1e9, 3) == 0.134
    assert round(A.workload_flops(8, 2048, 768, 3072, True) / 1e9, 1) == 283.5
    assert round(A.workload_flops(64, 1024, 1024, 4096, True) / 1e12, 3) == 1.787
    assert round(A.workload_flops(1, 131072, 2048, 8192, True) / 1e12, 2) == 83.56
    assert round(A.workload_flops(1, 32768, 4096, 16384, True, 4) / 1e12, 2) == 87.96


@pytest.mark.parametrize("n", [1, 7, 64, 130, 257])
@pytest.mark.parametrize("mask", [dict(), dict(window=1), dict(window=5), dict(window=64),
                                  dict(window=1000), dict(chunk=1), dict(chunk=3), dict(chunk=16),
                                  dict(chunk=1000)])
def test_visible_pairs_count_by_brute_force(n, mask):
    w, c = mask.get("window", 0), mask.get("chunk", 0)
    count = 0
    for p in range(n):
        for j in range(n):
            if c:
                count += j // c <= p // c
            else:
                count += j <= p and (not w or j > p - w)
    assert A.visible_pairs(n, True, **mask) == count
    assert A.visible_pairs(n, False) == n * n


def test_projection_flops_with_grouped_kv_heads():
    n, d = 1000, 1024
    assert A.projection_flops(n, d) == 8 * n * d * d
    assert A.projection_flops(n, d, 256) == 4 * n * d * d + 4 * n * d * 256
    assert A.layer_flops(n, d, 4 * d, True, d_kv=d) == A.layer_flops(n, d, 4 * d, True)


def test_layer_bwd_flops_closed_form():
    """Backward without recompute: 48 N d^2 dense at d_ff = 4d (twice the forward's
    24 N d^2) plus 2.5 times the attention's 2 d N (N + 1) (causal)."""
    n, d = 1024, 1024
    assert A.layer_bwd_flops(n, d, 4 * d, True) == 48 * n * d * d + 5 * d * n * (n + 1)
    assert A.layer_bwd_flops(n, d, 4 * d, False) == 48 * n * d * d + 10 * n * n * d
