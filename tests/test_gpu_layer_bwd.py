"""GPU parity of the layer backward (bpt_layer_bwd) against the oracle's
layer_backward.

Flow: the library's forward writes lse (bpt_layer_fwd_lse) for seeded bf16 X and
weights; bpt_layer_bwd then takes X, the weights, that lse and a seeded fp32 dZ.
The oracle computes every gradient in fp64 from X, the weights and dZ alone.

Small cases compare every element of dX and of every parameter gradient, with
ragged sequence lengths, both head sizes, both masks, and a d_ff wide enough
that the FFN runs over several row blocks (one of them ragged). The full-size case
is the 64 x 1024-token, d_model 1024 layer the forward is measured on: sequences
are independent, so (a) with dZ kept on two sequences only, every weight gradient
equals the oracle's over those two sequences and dX is exactly zero elsewhere;
(b) with dZ everywhere, dX of two sampled sequences equals the oracle's for those
sequences; (c) a second call gives identical bits (fixed summation order).

Tolerance: every product takes bf16 operands (activations and gradients rounded
to bf16 where they enter a product, 2^-9 relative, about 1.1e-3 rms each) with
fp32 accumulation. The longest chain (dZ -> dU -> dLN2 -> dY -> dA -> P, dS in the
attention backward -> dQ -> dLN1 -> dX) passes through about eight such roundings
in series, about sqrt(8) x 1.1e-3 = 3e-3 rms relative, on top of the recomputed
forward's own error (5e-3 on Z). Bound: relative Frobenius error 1e-2 per
gradient, and max |err| 3e-2 times the largest reference magnitude.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from blockwise_attn_ffn_amd import bpt, synth
from _parity import say, to_device

pytestmark = pytest.mark.gpu

REL_FRO, ABS = 1e-2, 3e-2
GRAD_KEYS = synth.LAYER_KEYS
# oracle names of the gradients (pages' (in, out) orientation for matrices)
ORACLE_KEY = {"ln1_g": "dln1_g", "ln1_b": "dln1_b", "w_q": "dw_q", "w_k": "dw_k", "w_v": "dw_v",
              "w_o": "dw_o", "ln2_g": "dln2_g", "ln2_b": "dln2_b", "w_1": "dw_1", "w_2": "dw_2"}


def run_fwd_bwd(w: synth.Workload, inputs: dict, dz: torch.Tensor, repeat: int = 1):
    """Forward (for lse), then the backward `repeat` times; returns (dX, grads) of each
    call on the host."""
    dev = to_device(inputs)
    layer = dev["layers"][0]
    desc = bpt.desc_for(w, out_dtype="f32")
    z = torch.empty((w.rows, w.d_model), dtype=torch.float32, device="cuda")
    lse = torch.full((w.batch, w.n_heads, w.seq_len), float("nan"), dtype=torch.float32, device="cuda")
    ws = bpt.alloc_workspace(bpt.layer_workspace_bytes(desc))
    bpt.layer_fwd_lse(desc, dev["x"], layer, z, lse, ws)
    del ws
    bws = bpt.alloc_workspace(bpt.layer_bwd_workspace_bytes(desc))
    dzd = dz.cuda()
    outs = []
    for _ in range(repeat):
        dx = torch.full((w.rows, w.d_model), float("nan"), dtype=torch.float32, device="cuda")
        grads = {k: torch.full(layer[k].shape, float("nan"), dtype=torch.float32, device="cuda")
                 for k in GRAD_KEYS}
        bpt.layer_bwd(desc, dev["x"], layer, lse, dzd, dx, grads, bws)
        torch.cuda.synchronize()
        outs.append((dx.cpu(), {k: t.cpu() for k, t in grads.items()}))
    return outs


def oracle_grads(w: synth.Workload, inputs: dict, dz: torch.Tensor, seqs=None) -> dict:
    """The oracle's gradients over the listed sequences (all if None): dX of those
    sequences stacked in order, parameter gradients summed over them, matrices in the
    library's [out, in] layout."""
    x = synth.to_f64(inputs["x"])
    d = synth.to_f64(dz)
    if seqs is not None:
        take = np.concatenate([np.arange(s * w.seq_len, (s + 1) * w.seq_len) for s in seqs])
        x, d = x[take], d[take]
    p = synth.oracle_weights(inputs["layers"][0])
    g = oracle.layer_backward(x, p, d, seq_len=w.seq_len, n_heads=w.n_heads, causal=w.causal,
                              eps=w.ln_eps, window=w.window, chunk=w.chunk)
    out = {"dx": g["dx"]}
    for k in GRAD_KEYS:
        a = g[ORACLE_KEY[k]]
        out[k] = a.T if a.ndim == 2 else a
    return out


def check(got, ref, what, floor=0.0):
    """floor: least scale of the max |err| bound (for gradients that vanish in exact
    arithmetic: with one token per sequence the softmax is constant in q, dW_Q = 0, and
    the computed value is rounding noise of the terms that cancel)."""
    got = got.double().numpy() if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    mx = oracle.max_abs_err(got, ref)
    fro = oracle.rel_fro_err(got, ref)
    scale = max(float(np.max(np.abs(ref))) if ref.size else 1.0, floor)
    say(f"  {what}: max|err| {mx:.3e} (|ref| <= {scale:.3g}), rel fro {fro:.3e}")
    assert mx <= ABS * scale and fro <= REL_FRO, what


def check_all(dx, grads, ref, tag):
    check(dx, ref["dx"], f"{tag} dX")
    floor = 1e-3 * max(float(np.max(np.abs(ref[k]))) for k in GRAD_KEYS)
    for k in GRAD_KEYS:
        check(grads[k], ref[k], f"{tag} d{k}", floor)


SMALL = [
    # name, batch, seq_len, d_model, n_heads, d_ff, causal
    ("dk64_causal_ragged", 2, 200, 256, 4, 1024, True),
    ("dk128_full_ragged", 1, 130, 256, 2, 512, False),
    ("one_token", 3, 1, 256, 4, 512, True),
    ("ffn_two_blocks", 1, 1100, 256, 2, 65536, True),   # blocks of 2^26 / d_ff = 1024 rows: 1024 + 76
    ("split_k", 2, 1100, 256, 4, 4096, True),           # dW_1, dW_2 over 2 row layers, dW_O, dW_QKV over 8
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_layer_bwd_small_every_element(case):
    name, batch, n, d, h, f, causal = case
    w = synth.Workload(name, batch=batch, seq_len=n, d_model=d, n_heads=h, d_ff=f, causal=causal,
                       block_q=128, block_kv=128, dtype="bf16", ln_random=True, w_std=0.08)
    inputs = synth.make_inputs(w, seed=11)
    dz = synth.make_grad_output(w.rows, d, seed=11)
    say(f"layer_bwd {name}: batch {batch} seq {n} d {d} heads {h} d_ff {f} causal {causal}")
    (dx, grads), = run_fwd_bwd(w, inputs, dz)
    check_all(dx, grads, oracle_grads(w, inputs, dz), name)


MASKED = [
    # name, batch, seq_len, d_model, n_heads, d_ff, window, chunk, n_kv_heads
    ("window_dk64", 2, 200, 256, 4, 1024, 100, 0, 0),
    ("chunk_dk64", 1, 300, 256, 4, 1024, 0, 96, 0),
    ("gqa2_dk64", 2, 200, 256, 4, 1024, 0, 0, 2),
    ("mqa_dk128", 1, 257, 256, 2, 512, 0, 0, 1),
    ("window_gqa2_dk128", 1, 300, 512, 4, 1024, 64, 0, 2),
]


@pytest.mark.parametrize("case", MASKED, ids=[c[0] for c in MASKED])
def test_layer_bwd_masks_and_kv_heads(case):
    """Every element against the oracle with a window, a chunked mask and fewer
    key/value heads (W_K, W_V and their gradients [n_kv_heads d_k, d_model]), ragged
    lengths. Weights of std 0.08 sqrt(256 / d_model), so that the projections (and
    the scores' spread) match the d_model 256 cases: the relative error of the bf16
    backward grows with the scores' spread (d_model 512 at std 0.08: ~1.1e-2 with no
    mask and all heads, as with the mask and grouped heads)."""
    name, batch, n, d, h, f, window, chunk, g = case
    w = synth.Workload(name, batch=batch, seq_len=n, d_model=d, n_heads=h, d_ff=f, causal=True,
                       block_q=128, block_kv=128 if d // h == 64 else 64, dtype="bf16", ln_random=True,
                       w_std=0.08 * math.sqrt(256 / d), window=window, chunk=chunk, n_kv_heads=g)
    inputs = synth.make_inputs(w, seed=13)
    dz = synth.make_grad_output(w.rows, d, seed=13)
    say(f"layer_bwd {name}: batch {batch} seq {n} d {d} heads {h}/{g or h} window {window} chunk {chunk}")
    (dx, grads), = run_fwd_bwd(w, inputs, dz)
    check_all(dx, grads, oracle_grads(w, inputs, dz), name)


def test_layer_bwd_full_size_sampled_sequences():
    """64 sequences of 1024 tokens, d_model 1024, 16 heads, d_ff 4096, causal."""
    w = synth.WORKLOADS["gpt2_medium"]
    inputs = synth.make_inputs(w, seed=0)
    seqs = [5, 62]
    live = np.concatenate([np.arange(s * w.seq_len, (s + 1) * w.seq_len) for s in seqs])
    # (a) dZ on two sequences only: weight gradients are those two sequences' sums
    dz = synth.make_grad_output(w.rows, w.d_model, seed=3, live_rows=live)
    say(f"layer_bwd full size (a): {w.name}, dZ on sequences {seqs}")
    (dx, grads), = run_fwd_bwd(w, inputs, dz)
    ref = oracle_grads(w, inputs, dz, seqs=seqs)
    dead = np.setdiff1d(np.arange(w.rows), live)
    assert torch.count_nonzero(dx[torch.from_numpy(dead)]).item() == 0, "dX nonzero where dZ is zero"
    check_all(dx[torch.from_numpy(live)], grads, ref, "full(a)")
    # (b) dZ everywhere: dX of the sampled sequences; (c) repeat calls are bit-identical
    dz = synth.make_grad_output(w.rows, w.d_model, seed=4)
    say(f"layer_bwd full size (b): {w.name}, dZ everywhere, checking sequences {seqs}")
    (dx1, g1), (dx2, g2) = run_fwd_bwd(w, inputs, dz, repeat=2)
    ref = oracle_grads(w, inputs, dz, seqs=seqs)
    check(dx1[torch.from_numpy(live)], ref["dx"], "full(b) dX")
    assert torch.equal(dx1, dx2), "dX differs between two calls"
    for k in GRAD_KEYS:
        assert torch.equal(g1[k], g2[k]), f"d{k} differs between two calls"


def test_layer_bwd_long_context_prefix():
    """The long-context layer: 1 x 131072 tokens, d_model 2048, 16 heads of 128,
    d_ff 8192, causal (query blocks of 128, key blocks of 64, 16 FFN blocks of 8192
    rows). With dZ kept on the first 768 rows only, the causal mask makes the whole
    backward that of the 768-token prefix (row i reaches only outputs j >= i, and
    the prefix's forward reads no later row): every parameter gradient and dX of the
    prefix equal the oracle's backward of the prefix, and dX is exactly zero past it."""
    w = synth.WORKLOADS["long_128k"]
    inputs = synth.make_inputs(w, seed=0)
    m = 768
    dz = synth.make_grad_output(w.rows, w.d_model, seed=5, live_rows=np.arange(m))
    say(f"layer_bwd long context: {w.name}, dZ on rows [0, {m})")
    (dx, grads), = run_fwd_bwd(w, inputs, dz)
    assert torch.count_nonzero(dx[m:]).item() == 0, "dX nonzero past the rows dZ reaches"
    p = synth.oracle_weights(inputs["layers"][0])
    g = oracle.layer_backward(synth.to_f64(inputs["x"][:m]), p, synth.to_f64(dz[:m]), seq_len=m,
                              n_heads=w.n_heads, causal=True, eps=w.ln_eps)
    ref = {"dx": g["dx"]}
    for k in GRAD_KEYS:
        a = g[ORACLE_KEY[k]]
        ref[k] = a.T if a.ndim == 2 else a
    check_all(dx[:m], grads, ref, "long(prefix)")
