"""The host (CPU) fused layer (bpt_layer_fwd_host) against the oracle: whole
layers on small shapes, fp32 arithmetic, so the fp32 bound (1e-4 max and
relative Frobenius) applies to fp32 and bf16 inputs alike (bf16 inputs are exact
in both). Runs without a GPU."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from blockwise_attn_ffn_amd import bpt, synth

TOL = 1e-4


def small(**kw) -> synth.Workload:
    base = dict(name="host", batch=2, seq_len=77, d_model=64, n_heads=4, d_ff=256, causal=True,
                block_q=32, block_kv=64, dtype="f32", ln_random=True, w_std=0.1)
    base.update(kw)
    return synth.Workload(**base)


def run_host(w, inp, out_dtype="f32", n_threads=3):
    desc = bpt.desc_for(w, out_dtype=out_dtype)
    nb = bpt.layer_host_workspace_bytes(desc, n_threads)
    assert nb > 0, bpt.last_error()
    ws = torch.empty(nb, dtype=torch.uint8)
    z = torch.full((w.rows, w.d_model), float("nan"), dtype=synth.TORCH_DTYPE[out_dtype])
    bpt.layer_fwd_host(desc, inp["x"], inp["layers"][0], z, ws, n_threads)
    return z


def oracle_z(w, inp):
    return oracle.layer_forward(synth.to_f64(inp["x"]), synth.oracle_weights(inp["layers"][0]),
                                seq_len=w.seq_len, n_heads=w.n_heads, causal=w.causal, eps=w.ln_eps,
                                window=w.window, chunk=w.chunk)


CASES = [dict(), dict(causal=False), dict(dtype="bf16"), dict(block_q=1), dict(block_q=128),
         dict(window=9), dict(chunk=10), dict(n_kv_heads=1), dict(n_kv_heads=2, window=30),
         dict(batch=1, seq_len=300, d_model=128, n_heads=2, d_ff=512, block_q=64),
         dict(seq_len=1), dict(d_model=72, n_heads=3, d_ff=200)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()) or "base")
def test_host_layer_matches_oracle(case):
    w = small(**case)
    inp = synth.make_inputs(w, seed=3)
    got = run_host(w, inp).double().numpy()
    ref = oracle_z(w, inp)
    assert oracle.max_abs_err(got, ref) < TOL and oracle.rel_fro_err(got, ref) < TOL


def test_host_layer_threads_and_bf16_output():
    """Each query block is one work item computed alone: any thread count gives the
    same bits; a bf16 Z is the round-to-nearest-even of the fp32 Z."""
    w = small(dtype="bf16", seq_len=200)
    inp = synth.make_inputs(w, seed=4)
    z1 = run_host(w, inp, n_threads=1)
    assert torch.equal(z1, run_host(w, inp, n_threads=5))
    assert torch.equal(run_host(w, inp, "bf16"), z1.to(torch.bfloat16))


def test_host_validation():
    w = small()
    d = bpt.desc_for(w)
    assert bpt.layer_host_workspace_bytes(d, 0) == 0
    d.d_model, d.n_heads = 60, 4          # d_head 15
    assert bpt.layer_host_workspace_bytes(d, 2) == 0 and "multiples of 8" in bpt.last_error()
    d = bpt.desc_for(w)
    d.precision = 1
    assert bpt.layer_host_workspace_bytes(d, 2) == 0
    d = bpt.desc_for(w)
    inp = synth.make_inputs(w, seed=5)
    z = torch.empty(w.rows, w.d_model)
    small_ws = torch.empty(16, dtype=torch.uint8)
    with pytest.raises(bpt.BptError, match="WORKSPACE"):
        bpt.layer_fwd_host(d, inp["x"], inp["layers"][0], z, small_ws, 2)
    ws = torch.empty(bpt.layer_host_workspace_bytes(d, 2), dtype=torch.uint8)
    with pytest.raises(bpt.BptError, match="ALIAS"):
        bpt.layer_fwd_host(d, inp["x"], inp["layers"][0], inp["x"], ws, 2)
