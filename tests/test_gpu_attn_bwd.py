"""GPU parity of the attention backward (bpt_attention_bwd) against the oracle.

Inputs are seeded bf16 Q, K, V, dO (synth.make_attention_inputs); the forward's
output O and statistic lse given to the library come from the oracle (O rounded to
bf16, lse to fp32), so every expected value is the oracle's. Small cases compare
every element; the full-size cases keep dO on a set of rows only (the gradient is
linear in dO), so that the oracle can evaluate dQ at those rows and dK, dV at
sampled keys one by one.

Tolerance: the kernels round P and dS to bf16 before their products (2^-9
relative each, round to nearest) and accumulate in fp32; D comes from O rounded to
bf16. The errors are those roundings summed over the keys (queries) with random
signs, so relative to the output's size they stay near 2^-9 / sqrt(terms): a
relative Frobenius bound of 5e-3 and an absolute bound of 2e-2 times the largest
reference magnitude (at least 1).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from blockwise_attn_ffn_amd import bpt, synth
from _parity import say

pytestmark = pytest.mark.gpu

REL_FRO, ABS = 5e-3, 2e-2


def fwd_stats(inp, batch, n, n_heads, causal, rows=None):
    """Oracle O (bf16) and lse (fp32 [batch, n_heads, n]) on the given global rows
    (all rows if None); other rows get O = 0, lse = 0 (their dO is zero)."""
    d = inp["q"].shape[1]
    q, k, v = (synth.to_f64(inp[x]) for x in ("q", "k", "v"))
    o = np.zeros((batch * n, d))
    lse = np.zeros((batch, n_heads, n))
    rows = np.arange(batch * n) if rows is None else np.asarray(rows, np.int64)
    for b in np.unique(rows // n):
        r = rows[rows // n == b]
        pos = r - b * n
        s0 = b * n
        o[r] = oracle.attention_sequence(q[s0 + pos], k[s0:s0 + n], v[s0:s0 + n], n_heads, causal,
                                         q_pos=pos)
        lse[b][:, pos] = oracle.attention_lse_sequence(q[s0 + pos], k[s0:s0 + n], n_heads, causal,
                                                       q_pos=pos)
    return (torch.from_numpy(o).to(torch.bfloat16),
            torch.from_numpy(lse).to(torch.float32))


def run_bwd(inp, o, lse, batch, n, n_heads, causal):
    d = inp["q"].shape[1]
    desc = bpt.make_attn_desc(batch=batch, seq_len=n, d_model=d, n_heads=n_heads, causal=causal)
    dev = {k: t.cuda() for k, t in inp.items()}
    outs = [torch.full((batch * n, d), float("nan"), dtype=torch.float32, device="cuda")
            for _ in range(3)]
    ws = bpt.alloc_workspace(bpt.attention_bwd_workspace_bytes(desc))
    bpt.attention_bwd(desc, dev["q"], dev["k"], dev["v"], o.cuda(), dev["do"], lse.cuda(), *outs, ws)
    torch.cuda.synchronize()
    return [t.cpu() for t in outs]


def check(got, ref, what):
    got = got.double().numpy() if isinstance(got, torch.Tensor) else got
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    mx = oracle.max_abs_err(got, ref)
    fro = oracle.rel_fro_err(got, ref)
    scale = max(1.0, float(np.max(np.abs(ref))) if ref.size else 1.0)
    say(f"  {what}: max|err| {mx:.3e} (|ref| <= {scale:.3g}), rel fro {fro:.3e}")
    assert mx <= ABS * scale and fro <= REL_FRO, what


SMALL = [
    # batch, seq_len, d_model, n_heads, causal, qk_std
    (1, 1, 64, 1, True, 1.0),
    (1, 1, 128, 1, False, 1.0),
    (2, 129, 128, 2, True, 1.0),
    (1, 300, 256, 2, False, 1.0),
    (2, 640, 256, 4, True, 1.0),
    (1, 1000, 512, 4, True, 2.0),
    (3, 200, 128, 1, False, 1.5),
    (1, 513, 256, 4, False, 0.5),
    (2, 700, 256, 2, True, 1.0),        # d_k 128, causal, two sequences, ragged last stage
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "b{}-n{}-d{}-h{}-c{}-s{}".format(*c))
def test_attention_bwd_small(case):
    batch, n, d, h, causal, qk_std = case
    say(f"case {case}")
    inp = synth.make_attention_inputs(batch, n, d, seed=7, qk_std=qk_std)
    o, lse = fwd_stats(inp, batch, n, h, causal)
    dq, dk, dv = run_bwd(inp, o, lse, batch, n, h, causal)
    for b in range(batch):
        r = slice(b * n, (b + 1) * n)
        ref = oracle.attention_backward_sequence(*(synth.to_f64(inp[x][r]) for x in ("q", "k", "v", "do")),
                                                 h, causal)
        for name, got, want in (("dQ", dq, ref[0]), ("dK", dk, ref[1]), ("dV", dv, ref[2])):
            check(got[r], want, f"{name} seq {b}")


def test_attention_bwd_single_token_closed_form():
    """One token: P = 1, so dV = dO and dQ = dK = 0 (dS = dP - D = 0)."""
    inp = synth.make_attention_inputs(1, 1, 128, seed=3)
    o, lse = fwd_stats(inp, 1, 1, 2, True)
    dq, dk, dv = run_bwd(inp, o, lse, 1, 1, 2, True)
    assert torch.equal(dv, inp["do"].float())
    assert float(dq.abs().max()) < 1e-5 and float(dk.abs().max()) < 1e-5


def _sampled(w, live, keys, seed):
    n, b = w.seq_len, w.batch
    inp = synth.make_attention_inputs(b, n, w.d_model, seed=seed, live_rows=live)
    o, lse = fwd_stats(inp, b, n, w.n_heads, w.causal, rows=live)
    say(f"case {w.name} attention backward, {live.size} live rows, {keys.size} keys")
    dq, dk, dv = run_bwd(inp, o, lse, b, n, w.n_heads, w.causal)
    dead = np.setdiff1d(np.arange(b * n), live)
    assert float(dq[torch.from_numpy(dead)].abs().max()) == 0.0, "dQ nonzero where dO is zero"
    for s in np.unique(live // n):
        r = slice(s * n, (s + 1) * n)
        q, k, v, g = (synth.to_f64(inp[x][r]) for x in ("q", "k", "v", "do"))
        lr = live[live // n == s] - s * n
        ref = oracle.attention_backward_dq_rows(q, k, v, g, w.n_heads, w.causal, lr)
        check(dq[s * n + lr], ref, f"dQ seq {s} live rows")
        kr = keys[keys // n == s] - s * n
        if kr.size:
            rk, rv = oracle.attention_backward_kv_rows(q, k, v, g, w.n_heads, w.causal, kr)
            check(dk[s * n + kr], rk, f"dK seq {s} sampled keys")
            check(dv[s * n + kr], rv, f"dV seq {s} sampled keys")
    return dk, dv, inp


def test_attention_bwd_gpt2_medium_shape():
    """64 sequences x 1024 tokens, 16 heads of 64: dO live on 48 rows of sequences 0,
    21, 42 and 63; dQ there and dK, dV at 48 keys of those sequences."""
    w = synth.WORKLOADS["gpt2_medium"]
    rng = np.random.default_rng(5)
    seqs = np.array([0, 21, 42, 63])
    live = np.sort(np.concatenate([s * w.seq_len + np.concatenate(
        [[0, 127, 128, 1023], rng.choice(np.arange(1, 1023), 8, replace=False)]) for s in seqs]))
    live = np.unique(live)
    keys = np.unique(np.concatenate([s * w.seq_len + np.concatenate(
        [[0, 1, 63, 64, 1022, 1023], rng.choice(1024, 6, replace=False)]) for s in seqs]))
    _sampled(w, live, keys, seed=11)


def test_attention_bwd_long_context_shape():
    """One sequence of 131072 tokens, 16 heads of 128: dO live on 40 rows; dQ there,
    dK and dV at 40 keys; and, at every key, the two identities that hold for any
    inputs: a head's dK sums to zero over the keys (rowsum dS = 0) and dV sums to the
    sum of dO (each softmax row sums to one)."""
    w = synth.WORKLOADS["long_128k"]
    n = w.seq_len
    rng = np.random.default_rng(9)
    live = np.unique(np.concatenate([[0, 63, 64, 127, 128, n // 2, n - 2, n - 1],
                                     rng.choice(n, 32, replace=False)]))
    keys = np.unique(np.concatenate([[0, 1, 127, 128, n // 2, n - 1], rng.choice(n, 34, replace=False)]))
    dk, dv, inp = _sampled(w, live, keys, seed=13)
    dkh = w.d_model // w.n_heads
    sum_dk = dk.double().sum(0).view(w.n_heads, dkh)
    fro_dk = dk.double().view(n, w.n_heads, dkh).pow(2).sum((0, 2)).sqrt()
    ratio = float((sum_dk.norm(dim=1) / fro_dk).max())
    say(f"  sum_k dK / |dK|_F per head: max {ratio:.3e}")
    assert ratio < 1e-2
    want = inp["do"].double().sum(0)
    err = float((dv.double().sum(0) - want).abs().max())
    say(f"  sum_k dV - sum_q dO: max {err:.3e} (|sum dO| <= {float(want.abs().max()):.3g})")
    assert err < 2e-2 * max(1.0, float(want.abs().max()))


VARIANTS = [
    # batch, seq_len, d_model, n_heads, mask / heads
    (2, 200, 256, 4, dict(window=37)),
    (1, 300, 256, 2, dict(window=100)),              # d_k 128
    (2, 257, 256, 4, dict(chunk=16)),
    (1, 400, 256, 2, dict(chunk=100)),
    (2, 200, 256, 4, dict(n_kv_heads=1)),
    (1, 333, 512, 4, dict(n_kv_heads=2)),            # d_k 128
    (2, 180, 256, 4, dict(n_kv_heads=2, window=50)),
    (1, 300, 512, 4, dict(n_kv_heads=1, chunk=64)),
    # d_k 128 over many 64-row query stages, a ragged last stage and two query heads
    # per key/value head (the split dK / dV kernel's grouped-head stage loop)
    (1, 2000, 512, 4, dict(n_kv_heads=2, window=300)),
    (1, 1500, 512, 4, dict(n_kv_heads=2, chunk=256)),
]


@pytest.mark.parametrize("case", VARIANTS, ids=lambda c: "b{}-n{}-d{}-h{}-".format(*c[:4]) +
                         "-".join(f"{k}{v}" for k, v in c[4].items()))
def test_attention_bwd_masks_and_grouped_heads(case):
    batch, n, d, h, var = case
    window, chunk, g = var.get("window", 0), var.get("chunk", 0), var.get("n_kv_heads", 0)
    dkv = (g or h) * (d // h)
    say(f"case {case}")
    inp = synth.make_attention_inputs(batch, n, d, seed=17)
    inp["k"] = inp["k"][:, :dkv].contiguous()
    inp["v"] = inp["v"][:, :dkv].contiguous()
    q, k, v = (synth.to_f64(inp[x]) for x in ("q", "k", "v"))
    o = np.zeros((batch * n, d))
    lse = np.zeros((batch, h, n))
    for b in range(batch):
        r = slice(b * n, (b + 1) * n)
        o[r] = oracle.attention_sequence(q[r], k[r], v[r], h, True, window=window, chunk=chunk)
        lse[b] = oracle.attention_lse_sequence(q[r], k[r], h, True, window=window, chunk=chunk)
    desc = bpt.make_attn_desc(batch=batch, seq_len=n, d_model=d, n_heads=h, causal=True,
                              window=window, chunk=chunk, n_kv_heads=g)
    dev = {x: t.cuda() for x, t in inp.items()}
    dq = torch.full((batch * n, d), float("nan"), device="cuda")
    dk = torch.full((batch * n, dkv), float("nan"), device="cuda")
    dv = torch.full((batch * n, dkv), float("nan"), device="cuda")
    ws = bpt.alloc_workspace(bpt.attention_bwd_workspace_bytes(desc))
    bpt.attention_bwd(desc, dev["q"], dev["k"], dev["v"], torch.from_numpy(o).to(torch.bfloat16).cuda(),
                      dev["do"], torch.from_numpy(lse).float().cuda(), dq, dk, dv, ws)
    torch.cuda.synchronize()
    for b in range(batch):
        r = slice(b * n, (b + 1) * n)
        ref = oracle.attention_backward_sequence(q[r], k[r], v[r], synth.to_f64(inp["do"][r]), h, True,
                                                 window=window, chunk=chunk)
        for name, got, want in (("dQ", dq, ref[0]), ("dK", dk, ref[1]), ("dV", dv, ref[2])):
            check(got.cpu()[r], want, f"{name} seq {b}")
