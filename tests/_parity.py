"""Helpers shared by the GPU parity tests: run the library on seeded inputs and
evaluate the oracle on the same values."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from blockwise_attn_ffn_amd import bpt, synth

# Tolerances: max |err| and relative Frobenius error of Z against the oracle.
TOL = {"bf16": (2e-2, 5e-3), "f32": (1e-4, 1e-4)}


def say(*a):
    """Name the case before a GPU step, flushed, so a failing run shows it."""
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(inputs: dict, device="cuda") -> dict:
    return {"x": inputs["x"].to(device),
            "layers": [{k: v.to(device) for k, v in l.items()} for l in inputs["layers"]]}


def run_gpu(w: synth.Workload, inputs: dict, out_dtype: str = "f32") -> torch.Tensor:
    """Run the layer (or stack) through the C ABI; returns Z on the host."""
    dev = to_device(inputs)
    desc = bpt.desc_for(w, out_dtype=out_dtype)
    z = torch.empty((w.rows, w.d_model), dtype=synth.TORCH_DTYPE[out_dtype], device="cuda")
    if w.n_layers == 1:
        ws = bpt.alloc_workspace(bpt.layer_workspace_bytes(desc))
        bpt.layer_fwd(desc, dev["x"], dev["layers"][0], z, ws)
    else:
        ws = bpt.alloc_workspace(bpt.stack_workspace_bytes(desc, w.n_layers))
        bpt.stack_fwd(desc, dev["x"], dev["layers"], z, ws)
    torch.cuda.synchronize()
    return z.cpu()


def run_gpu_lse(w: synth.Workload, inputs: dict, out_dtype: str = "f32"):
    """One layer through bpt_layer_fwd_lse; returns (Z, lse [batch, n_heads, seq_len]) on
    the host."""
    assert w.n_layers == 1
    dev = to_device(inputs)
    desc = bpt.desc_for(w, out_dtype=out_dtype)
    z = torch.empty((w.rows, w.d_model), dtype=synth.TORCH_DTYPE[out_dtype], device="cuda")
    lse = torch.full((w.batch, w.n_heads, w.seq_len), float("nan"), dtype=torch.float32, device="cuda")
    ws = bpt.alloc_workspace(bpt.layer_workspace_bytes(desc))
    bpt.layer_fwd_lse(desc, dev["x"], dev["layers"][0], z, lse, ws)
    torch.cuda.synchronize()
    return z.cpu(), lse.cpu()


# Tolerance of the attention statistic lse (natural log, absolute): the scores it
# sums carry the rounding of the computed operands Q and K (bf16: 2^-9 relative
# each, pairs: ~2^-17), so its error is of the order of that relative error times
# the scores' size; the bound is the Z bound's magnitude for bf16.
LSE_TOL = {"bf16": 2e-2, "pairs": 1e-5, "f32": 1e-4}


def check_lse(got: torch.Tensor, ref: np.ndarray, kind: str, what: str = "") -> float:
    g = got.to(torch.float64).numpy()
    assert np.all(np.isfinite(g)), f"{what}: non-finite lse"
    mx = float(np.max(np.abs(g - ref)))
    say(f"  {what}: lse max|err| = {mx:.3e} (tol {LSE_TOL[kind]:g})")
    assert mx <= LSE_TOL[kind], what
    return mx


def oracle_full(w: synth.Workload, inputs: dict, seqs=None) -> np.ndarray:
    """Oracle Z of every row (or of the listed sequences, stacked in order)."""
    x = synth.to_f64(inputs["x"])
    if seqs is not None:
        x = np.concatenate([x[s * w.seq_len:(s + 1) * w.seq_len] for s in seqs])
    layers = [synth.oracle_weights(l) for l in inputs["layers"]]
    return oracle.stack_forward(x, layers, seq_len=w.seq_len, n_heads=w.n_heads,
                                causal=w.causal, eps=w.ln_eps, window=w.window, chunk=w.chunk)


def oracle_rows(w: synth.Workload, inputs: dict, rows: np.ndarray) -> np.ndarray:
    x = synth.to_f64(inputs["x"])
    layers = [synth.oracle_weights(l) for l in inputs["layers"]]
    return oracle.stack_forward_rows(x, layers, rows, seq_len=w.seq_len, n_heads=w.n_heads,
                                     causal=w.causal, eps=w.ln_eps, window=w.window, chunk=w.chunk)


def seq_rows(w: synth.Workload, seqs) -> np.ndarray:
    return np.concatenate([np.arange(s * w.seq_len, (s + 1) * w.seq_len) for s in seqs])


def check(got: torch.Tensor | np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    g = got.to(torch.float64).numpy() if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    mx = oracle.max_abs_err(g, ref)
    rf = oracle.rel_fro_err(g, ref)
    tmax, tfro = TOL[dtype]
    say(f"  {what}: max|err| = {mx:.3e} (tol {tmax:g}), rel fro = {rf:.3e} (tol {tfro:g})")
    assert mx <= tmax and rf <= tfro, f"{what}: max|err| {mx:.3e}, rel fro {rf:.3e}"
    return mx, rf
