"""GPU parity of the attention masks of the transformer-cost page's Section 5 — the
windowed mask (query p reads keys p - w + 1 .. p) and chunked streaming (query p
reads its whole chunk and the earlier ones) — through the whole layer, on every
attention kernel path, against the oracle; plus the saved statistic under both
masks and the 131072-token layer with a 4096-token window on sampled rows."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from blockwise_attn_ffn_amd import synth
from _parity import check, check_lse, oracle_full, oracle_rows, run_gpu, run_gpu_lse, say

pytestmark = pytest.mark.gpu


def small(**kw) -> synth.Workload:
    base = dict(name="small_mask", batch=2, seq_len=200, d_model=256, n_heads=4, d_ff=1024,
                causal=True, block_q=128, block_kv=128, dtype="bf16", ln_random=True)
    base.update(kw)
    return synth.Workload(**base)


CASES = [
    # d_k 64, one-group kernel
    dict(window=1),
    dict(window=100, block_q=64, block_kv=64),
    dict(window=130, block_q=128, block_kv=64, seq_len=640),
    dict(chunk=1),
    dict(chunk=16),
    dict(chunk=100, block_q=64, block_kv=128, seq_len=513),
    # d_k 128: two-group kernel (block_q 128), one-group (block_q 64)
    dict(n_heads=2, window=37, block_kv=64, seq_len=640),
    dict(n_heads=2, window=300, block_kv=128, seq_len=1000, batch=1),
    dict(n_heads=2, window=129, block_q=64, block_kv=64, seq_len=400),
    dict(n_heads=2, window=5000, block_kv=64),                     # longer than the sequence
    dict(n_heads=2, chunk=100, block_kv=64, seq_len=640),
    dict(n_heads=2, chunk=1000, block_kv=128),                     # one chunk: no mask
    # fp32 and bf16 pairs
    dict(dtype="f32", d_model=128, n_heads=2, d_ff=512, block_q=64, block_kv=64, window=50),
    dict(dtype="f32", d_model=128, n_heads=2, d_ff=512, block_q=64, block_kv=64, chunk=24),
    dict(window=80, precision=1),
    dict(n_heads=2, chunk=48, precision=1, block_kv=64),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_masked_layer_small(case):
    w = small(**case)
    say(f"case {w}")
    inp = synth.make_inputs(w, seed=21)
    got = run_gpu(w, inp, "f32")
    check(got, oracle_full(w, inp), "f32" if w.dtype == "f32" else "bf16", f"{case}")


def test_chunk_one_equals_causal_and_whole_chunk_equals_unmasked():
    """Chunk 1 is the plain causal mask and a chunk of the whole length is no mask:
    the library gives bit-identical Z for the equivalent descriptors."""
    w = small(n_heads=2, block_kv=64, seq_len=300)
    inp = synth.make_inputs(w, seed=23)
    say("case chunk 1 / chunk N equivalences")
    assert torch.equal(run_gpu(w.replace(chunk=1), inp), run_gpu(w, inp))
    full = run_gpu(w.replace(causal=False), inp)
    assert torch.equal(run_gpu(w.replace(chunk=300), inp), full)


@pytest.mark.parametrize("case", [dict(window=70), dict(n_heads=2, window=200, block_kv=64, seq_len=640),
                                  dict(chunk=32), dict(n_heads=2, chunk=96, block_kv=64)],
                         ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_masked_lse(case):
    w = small(**case)
    say(f"case {w}")
    inp = synth.make_inputs(w, seed=25)
    _, lse = run_gpu_lse(w, inp)
    ref = oracle.layer_lse(synth.to_f64(inp["x"]), synth.oracle_weights(inp["layers"][0]),
                           seq_len=w.seq_len, n_heads=w.n_heads, causal=True, eps=w.ln_eps,
                           window=w.window, chunk=w.chunk)
    check_lse(lse, ref, "bf16", f"lse {case}")


def test_long_context_window_4096_sampled_rows():
    w = synth.WORKLOADS["long_128k_w4096"]
    say(f"case {w}")
    inp = synth.make_inputs(w, seed=0)
    got = run_gpu(w, inp, "f32")
    rows = synth.sample_rows(w, w.sample_rows, seed=0)
    check(got[torch.from_numpy(rows)], oracle_rows(w, inp, rows), "bf16", w.name)
