"""GPU parity of grouped-query attention (the transformer-cost page's MQA and GQA:
g key/value heads, query head h reads head h / (n_heads / g)) through the whole
layer, on every attention kernel path and both epilogues, against the oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from blockwise_attn_ffn_amd import synth
from _parity import check, check_lse, oracle_full, oracle_rows, run_gpu, run_gpu_lse, say

pytestmark = pytest.mark.gpu


def small(**kw) -> synth.Workload:
    base = dict(name="small_gqa", batch=2, seq_len=200, d_model=256, n_heads=4, d_ff=1024,
                causal=True, block_q=128, block_kv=128, dtype="bf16", ln_random=True)
    base.update(kw)
    return synth.Workload(**base)


CASES = [
    dict(n_kv_heads=1),                                             # MQA, d_k 64, one-group
    dict(n_kv_heads=2, block_q=64, block_kv=64, seq_len=300),
    dict(n_kv_heads=2, window=50, block_kv=64),                    # with a window
    dict(n_kv_heads=1, n_heads=2, block_kv=64, seq_len=640),        # d_k 128, two-group
    dict(n_kv_heads=2, d_model=512, n_heads=4, d_ff=2048, block_kv=128, seq_len=500, chunk=64),
    dict(n_kv_heads=1, n_heads=2, block_q=64, block_kv=64, seq_len=400),   # d_k 128, one-group
    dict(n_kv_heads=4, d_model=1024, n_heads=16, d_ff=4096, seq_len=300, causal=False),
    dict(dtype="f32", d_model=128, n_heads=2, d_ff=512, block_q=64, block_kv=64, n_kv_heads=1),
    dict(n_kv_heads=2, precision=1),                                # bf16 pairs, staged
    dict(n_kv_heads=2, d_model=2048, n_heads=16, d_ff=8192, block_kv=64, seq_len=300),  # staged, Y room
    dict(n_kv_heads=1, d_model=2048, n_heads=16, d_ff=8192, block_kv=64, seq_len=260, batch=1),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_gqa_layer_small(case):
    w = small(**case)
    say(f"case {w}")
    inp = synth.make_inputs(w, seed=31)
    assert inp["layers"][0]["w_k"].shape == (w.d_kv, w.d_model)
    got = run_gpu(w, inp, "f32")
    check(got, oracle_full(w, inp), "f32" if w.dtype == "f32" else "bf16", f"{case}")


def test_gqa_with_all_heads_equals_multi_head():
    """n_kv_heads = n_heads is multi-head attention: bit-identical to n_kv_heads = 0."""
    w = small(n_heads=2, block_kv=64, seq_len=300)
    inp = synth.make_inputs(w, seed=33)
    say("case n_kv_heads = n_heads")
    assert torch.equal(run_gpu(w.replace(n_kv_heads=2), inp), run_gpu(w, inp))


@pytest.mark.parametrize("case", [dict(n_kv_heads=1), dict(n_kv_heads=1, n_heads=2, block_kv=64, seq_len=640)],
                         ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_gqa_lse(case):
    w = small(**case)
    say(f"case {w}")
    inp = synth.make_inputs(w, seed=35)
    _, lse = run_gpu_lse(w, inp)
    ref = oracle.layer_lse(synth.to_f64(inp["x"]), synth.oracle_weights(inp["layers"][0]),
                           seq_len=w.seq_len, n_heads=w.n_heads, causal=True, eps=w.ln_eps)
    check_lse(lse, ref, "bf16", f"lse {case}")


def test_gqa_long_context_sampled_rows():
    """The 131072-token layer with 4 key/value heads for its 16 query heads."""
    w = synth.WORKLOADS["long_128k_gqa4"]
    say(f"case {w}")
    inp = synth.make_inputs(w, seed=0)
    got = run_gpu(w, inp, "f32")
    rows = synth.sample_rows(w, w.sample_rows, seed=0)
    check(got[torch.from_numpy(rows)], oracle_rows(w, inp, rows), "bf16", w.name)
