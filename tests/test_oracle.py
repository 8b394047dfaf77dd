"""Pins of the CPU oracle against things other than itself (no GPU needed).

Each test names what fixes the expected value: a number or identity printed on
the pages, a closed form, a brute-force loop on tiny inputs, or an independent
library routine (torch's CPU float64 functional ops, scipy).
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle
from oracle import bpt_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_layer(rng, d, d_ff, std=0.2, ln_random=True):
    """float64 weights in (in, out) orientation for tiny oracle-only checks."""
    g = lambda *s: rng.standard_normal(s)  # noqa: E731
    p = dict(w_q=g(d, d) * std, w_k=g(d, d) * std, w_v=g(d, d) * std, w_o=g(d, d) * std,
             w_1=g(d, d_ff) * std, w_2=g(d_ff, d) * std)
    if ln_random:
        p.update(ln1_g=1 + 0.1 * g(d), ln1_b=0.1 * g(d), ln2_g=1 + 0.1 * g(d), ln2_b=0.1 * g(d))
    else:
        p.update(ln1_g=np.ones(d), ln1_b=np.zeros(d), ln2_g=np.ones(d), ln2_b=np.zeros(d))
    return p


# --------------------------------------------------------------------------
# Online softmax: the pages' two-tile running-sum example, generalised
# --------------------------------------------------------------------------

def test_two_tile_running_sum_prints_true():
    """transformer-cost page, FlashAttention paragraph: 8 scores in two tiles of 4; the
    rescaled tile sums equal the full sum (the page prints True)."""
    g = json.load(open(os.path.join(GOLDEN, "pages_numbers.json")))["two_tile_running_sum"]
    rng = np.random.default_rng(0)
    for _ in range(50):
        s = rng.standard_normal(g["scores"])
        m, l, _o = oracle.online_softmax_tiles(s, np.ones((s.size, 1)), g["tile"])
        full = np.exp(s - s.max()).sum()            # the page's "full" line
        assert m == s.max()
        assert bool(np.allclose(l, full)) is g["printed"]


@pytest.mark.parametrize("n,tile", [(8, 4), (37, 5), (64, 64), (100, 7), (3, 10)])
def test_online_softmax_accumulator_matches_scipy_softmax(n, tile):
    """The (m, l, o) recurrence with o/l equals scipy's softmax-weighted mean, for any
    number of tiles and a ragged last tile."""
    rng = np.random.default_rng(n * 31 + tile)
    s = rng.standard_normal(n) * 4
    v = rng.standard_normal((n, 6))
    m, l, o = oracle.online_softmax_tiles(s, v, tile)
    ref = scipy.special.softmax(s) @ v
    assert np.max(np.abs(o / l - ref)) < 1e-13
    assert abs(l - np.exp(s - s.max()).sum()) < 1e-12 * l


def test_online_softmax_leading_masked_tile_and_peaky_scores():
    """A first tile with every score -inf leaves the state untouched; huge scores do not
    overflow because the running maximum is subtracted."""
    s = np.array([-np.inf] * 4 + [1000.0, 999.0, -3.0, 0.5])
    v = np.arange(16, dtype=float).reshape(8, 2)
    m, l, o = oracle.online_softmax_tiles(s, v, 4)
    ref = scipy.special.softmax(s[4:]) @ v[4:]
    assert m == 1000.0 and np.allclose(o / l, ref, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# Attention: brute force and an independent library routine
# --------------------------------------------------------------------------

def brute_force_attention(q, k, v, n_heads, causal):
    """Explicit loops over head, query and key with math.exp and one division."""
    nq, d = q.shape
    dk = d // n_heads
    out = np.zeros((nq, d))
    for h in range(n_heads):
        for i in range(nq):
            keys = range(i + 1) if causal else range(k.shape[0])
            sc = {j: sum(q[i, h * dk + c] * k[j, h * dk + c] for c in range(dk)) / math.sqrt(dk)
                  for j in keys}
            mx = max(sc.values())
            w = {j: math.exp(sc[j] - mx) for j in keys}
            tot = sum(w.values())
            for c in range(dk):
                out[i, h * dk + c] = sum(w[j] * v[j, h * dk + c] for j in keys) / tot
    return out


@pytest.mark.parametrize("causal", [False, True])
def test_attention_matches_brute_force(causal):
    rng = np.random.default_rng(1 + causal)
    n, d, h = 9, 8, 2
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    got = oracle.attention_sequence(q, k, v, h, causal)
    assert np.max(np.abs(got - brute_force_attention(q, k, v, h, causal))) < 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_attention_matches_torch_sdpa(causal):
    rng = np.random.default_rng(7 + causal)
    n, d, h = 50, 32, 4
    q, k, v = (rng.standard_normal((n, d)) * 2 for _ in range(3))
    got = oracle.attention_sequence(q, k, v, h, causal)
    t = lambda a: torch.from_numpy(a).view(n, h, d // h).transpose(0, 1).contiguous()  # noqa: E731
    ref = F.scaled_dot_product_attention(t(q)[None], t(k)[None], t(v)[None], is_causal=causal)
    ref = ref[0].transpose(0, 1).reshape(n, d).numpy()
    assert np.max(np.abs(got - ref)) < 1e-12


def test_attention_sampled_positions_match_full():
    """Queries at arbitrary positions see exactly the keys up to their position."""
    rng = np.random.default_rng(3)
    n, d, h = 40, 16, 2
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    full = oracle.attention_sequence(q, k, v, h, True)
    pos = np.array([0, 5, 17, 39])
    part = oracle.attention_sequence(q[pos], k[:40], v[:40], h, True, q_pos=pos)
    assert np.max(np.abs(part - full[pos])) < 1e-14


@pytest.mark.parametrize("causal", [False, True])
def test_attention_query_chunks_match_brute_force(causal):
    """Evaluating query rows in groups (a memory bound) is checked against the
    brute-force loops, with ragged groups and sampled positions."""
    rng = np.random.default_rng(11 + causal)
    n, d, h = 23, 8, 2
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    ref = brute_force_attention(q, k, v, h, causal)
    for chunk in (1, 5, 22, 23, 64):
        got = oracle.attention_sequence(q, k, v, h, causal, q_chunk=chunk)
        assert np.max(np.abs(got - ref)) < 1e-13, chunk
    pos = np.array([2, 3, 11, 19, 22])
    got = oracle.attention_sequence(q[pos], k, v, h, causal, q_pos=pos, q_chunk=2)
    assert np.max(np.abs(got - ref[pos])) < 1e-13


def test_uniform_attention_closed_form():
    """W_Q = 0 makes every score 0: causal row p returns mean(V[0..p]); without the
    mask every row returns mean(V)."""
    rng = np.random.default_rng(4)
    n, d = 12, 8
    v = rng.standard_normal((n, d))
    q = np.zeros((n, d))
    k = rng.standard_normal((n, d))
    causal = oracle.attention_sequence(q, k, v, 2, True)
    assert np.allclose(causal, np.cumsum(v, 0) / np.arange(1, n + 1)[:, None], atol=1e-14)
    full = oracle.attention_sequence(q, k, v, 2, False)
    assert np.allclose(full, np.broadcast_to(v.mean(0), (n, d)), atol=1e-14)


def test_softmax_shift_invariance_and_masked_row():
    rng = np.random.default_rng(5)
    s = rng.standard_normal((4, 7))
    assert np.allclose(oracle.softmax_rows(s), oracle.softmax_rows(s + 123.0), atol=1e-15)
    assert np.all(oracle.softmax_rows(np.full((1, 3), -np.inf)) == 0)   # no NaN


# --------------------------------------------------------------------------
# LN and GELU: closed forms and torch
# --------------------------------------------------------------------------

def test_layer_norm_closed_forms_and_torch():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((5, 16)) * 3 + 2
    g, b = rng.standard_normal(16), rng.standard_normal(16)
    ref = F.layer_norm(torch.from_numpy(x), (16,), torch.from_numpy(g), torch.from_numpy(b), 1e-5)
    assert np.max(np.abs(oracle.layer_norm(x, g, b, 1e-5) - ref.numpy())) < 1e-13
    # a constant row normalises to the bias
    assert np.allclose(oracle.layer_norm(np.full((1, 16), 7.5), g, b, 1e-5), b, atol=0)
    # two-valued row a +- delta: entries are +- delta / sqrt(delta^2 + eps) (eps inside sqrt)
    delta, eps = 1e-3, 1e-5
    row = np.array([[5 + delta, 5 - delta] * 4])
    got = oracle.layer_norm(row, np.ones(8), np.zeros(8), eps)
    assert np.allclose(got[0, 0], delta / math.sqrt(delta * delta + eps), rtol=1e-12)


def test_gelu_tanh_values():
    u = np.linspace(-8, 8, 2001)
    ref = F.gelu(torch.from_numpy(u), approximate="tanh").numpy()
    assert np.max(np.abs(oracle.gelu_tanh(u) - ref)) < 1e-15
    # closed form at u = 1: 0.5 (1 + tanh(sqrt(2/pi) * 1.044715))
    assert abs(oracle.gelu_tanh(np.array([1.0]))[0]
               - 0.5 * (1 + math.tanh(math.sqrt(2 / math.pi) * 1.044715))) < 1e-15
    # the tanh form is not the erf form: a swap would be visible here
    erf_form = 0.5 * u * (1 + scipy.special.erf(u / math.sqrt(2)))
    assert np.max(np.abs(oracle.gelu_tanh(u) - erf_form)) > 1e-4


# --------------------------------------------------------------------------
# The whole layer: the pages' fused loop, torch, closed forms, row independence
# --------------------------------------------------------------------------

def torch_layer(x, p, seq_len, n_heads, causal, eps=1e-5):
    """The layer assembled from torch CPU float64 functional ops (layer_norm, matmul,
    scaled_dot_product_attention, gelu) -- a second, library-built implementation."""
    t = {k: torch.from_numpy(np.asarray(v, np.float64)) for k, v in p.items()}
    xt = torch.from_numpy(x)
    rows, d = xt.shape
    dk = d // n_heads
    x1 = F.layer_norm(xt, (d,), t["ln1_g"], t["ln1_b"], eps)
    split = lambda a: a.view(rows // seq_len, seq_len, n_heads, dk).transpose(1, 2)  # noqa: E731
    a = F.scaled_dot_product_attention(split(x1 @ t["w_q"]), split(x1 @ t["w_k"]),
                                       split(x1 @ t["w_v"]), is_causal=causal)
    a = a.transpose(1, 2).reshape(rows, d)
    y = xt + a @ t["w_o"]
    h = F.gelu(F.layer_norm(y, (d,), t["ln2_g"], t["ln2_b"], eps) @ t["w_1"], approximate="tanh")
    return (y + h @ t["w_2"]).numpy()


@pytest.mark.parametrize("causal", [False, True])
def test_layer_matches_torch_built_layer(causal):
    rng = np.random.default_rng(10 + causal)
    seq, b, d, h = 24, 2, 16, 4
    x = rng.standard_normal((seq * b, d))
    p = rand_layer(rng, d, 4 * d)
    got = oracle.layer_forward(x, p, seq_len=seq, n_heads=h, causal=causal)
    ref = torch_layer(x, p, seq, h, causal)
    assert np.max(np.abs(got - ref)) < 1e-12


@pytest.mark.parametrize("causal,seq,bq,bkv", [(False, 64, 16, 16), (True, 64, 16, 16),
                                                (True, 64, 32, 16), (True, 50, 16, 8),
                                                (False, 45, 32, 64), (True, 16, 16, 16)])
def test_fused_blockwise_loop_equals_unfused(causal, seq, bq, bkv):
    """The pages' fused loop (online softmax, causal block skip, K/V recomputed per block,
    ragged last blocks) gives the unfused layer's values up to rounding."""
    rng = np.random.default_rng(seq + bq + 3 * bkv + causal)
    d, h = 16, 2
    x = rng.standard_normal((2 * seq, d))
    p = rand_layer(rng, d, 4 * d, std=0.4)
    ref = oracle.layer_forward(x, p, seq_len=seq, n_heads=h, causal=causal)
    got = oracle.blockwise_layer_forward(x, p, seq_len=seq, n_heads=h, causal=causal,
                                         block_q=bq, block_kv=bkv)
    assert oracle.rel_fro_err(got, ref) < 1e-12


def test_layer_closed_forms():
    rng = np.random.default_rng(12)
    seq, d, h = 20, 16, 2
    x = rng.standard_normal((seq, d))
    p = rand_layer(rng, d, 64)
    # W_O = 0 -> Y = X; W_V = 0 -> attention output 0 -> Y = X
    for key in ("w_o", "w_v"):
        q = dict(p, **{key: np.zeros_like(p[key])})
        _z, parts = oracle.layer_forward(x, q, seq_len=seq, n_heads=h, causal=True, return_parts=True)
        assert np.array_equal(parts["y"], x)
    # W_2 = 0 -> Z = Y
    q = dict(p, w_2=np.zeros_like(p["w_2"]))
    z, parts = oracle.layer_forward(x, q, seq_len=seq, n_heads=h, causal=True, return_parts=True)
    assert np.array_equal(z, parts["y"])
    # W_Q = 0 -> causal row p of the attention output is mean(V[0..p]); here V = LN1(X) W_V
    q = dict(p, w_q=np.zeros_like(p["w_q"]))
    _z, parts = oracle.layer_forward(x, q, seq_len=seq, n_heads=h, causal=True, return_parts=True)
    vv = oracle.layer_norm(x, p["ln1_g"], p["ln1_b"], 1e-5) @ p["w_v"]
    assert np.allclose(parts["a"], np.cumsum(vv, 0) / np.arange(1, seq + 1)[:, None], atol=1e-13)


def test_row_independence_of_tail_and_noncausal_permutation():
    """LN, the FFN and the residuals are row-wise: permuting a non-causal sequence's rows
    permutes the outputs; a single row evaluated alone equals that row of the full layer."""
    rng = np.random.default_rng(13)
    seq, d, h = 30, 16, 4
    x = rng.standard_normal((seq, d))
    p = rand_layer(rng, d, 64)
    z = oracle.layer_forward(x, p, seq_len=seq, n_heads=h, causal=False)
    perm = rng.permutation(seq)
    zp = oracle.layer_forward(x[perm], p, seq_len=seq, n_heads=h, causal=False)
    assert np.max(np.abs(zp - z[perm])) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_rows_equal_full_rows(causal):
    rng = np.random.default_rng(14 + causal)
    seq, b, d, h = 33, 3, 16, 2
    x = rng.standard_normal((seq * b, d))
    p = rand_layer(rng, d, 64)
    z = oracle.layer_forward(x, p, seq_len=seq, n_heads=h, causal=causal)
    rows = np.array([0, 1, 32, 33, 34, 50, 65, 66, 98])
    got = oracle.layer_forward_rows(x, p, rows, seq_len=seq, n_heads=h, causal=causal, row_chunk=7)
    assert np.max(np.abs(got - z[rows])) < 1e-12


def test_stack_rows_and_single_layer_stack():
    rng = np.random.default_rng(15)
    seq, d, h = 24, 16, 2
    x = rng.standard_normal((2 * seq, d))
    layers = [rand_layer(rng, d, 64, std=0.2 / math.sqrt(2 * i + 1)) for i in range(3)]
    full = oracle.stack_forward(x, layers, seq_len=seq, n_heads=h, causal=True)
    step = x
    for p in layers:
        step = torch_layer(step, p, seq, h, True)
    assert np.max(np.abs(full - step)) < 1e-11
    rows = np.array([0, 5, 23, 24, 47])
    got = oracle.stack_forward_rows(x, layers, rows, seq_len=seq, n_heads=h, causal=True)
    assert np.max(np.abs(got - full[rows])) < 1e-12
    one = oracle.stack_forward(x, layers[:1], seq_len=seq, n_heads=h, causal=True)
    assert np.array_equal(one, oracle.layer_forward(x, layers[0], seq_len=seq, n_heads=h, causal=True))


# --------------------------------------------------------------------------
# Planted mistakes: each pin above must catch a plausible error in the oracle
# --------------------------------------------------------------------------

@pytest.mark.parametrize("mutation", ["scale_1_over_dk", "no_causal_mask", "erf_gelu",
                                      "transposed_wo", "no_second_residual", "ln_no_eps"])
def test_pins_catch_planted_oracle_mistakes(mutation, monkeypatch):
    rng = np.random.default_rng(16)
    seq, d, h = 24, 16, 2
    x = rng.standard_normal((seq, d))
    p = rand_layer(rng, d, 64, std=0.5)
    ref = torch_layer(x, p, seq, h, True, eps=1e-2)
    if mutation == "scale_1_over_dk":
        orig = O.attention_sequence

        def bad(q, k, v, n_heads, causal, q_pos=None, q_chunk=None, **kw):
            return orig(q * math.sqrt(d // n_heads) ** -1, k, v, n_heads, causal, q_pos, q_chunk, **kw)
        monkeypatch.setattr(O, "attention_sequence", bad)
    elif mutation == "no_causal_mask":
        orig = O.attention_sequence
        monkeypatch.setattr(O, "attention_sequence",
                            lambda q, k, v, n_heads, causal, q_pos=None, q_chunk=None, **kw:
                            orig(q, k, v, n_heads, False, q_pos, q_chunk))
    elif mutation == "erf_gelu":
        monkeypatch.setattr(O, "gelu_tanh", lambda u: 0.5 * u * (1 + scipy.special.erf(u / math.sqrt(2))))
    elif mutation == "transposed_wo":
        p = dict(p)
        ref = torch_layer(x, dict(p, w_o=p["w_o"].T.copy()), seq, h, True, eps=1e-2)
    elif mutation == "no_second_residual":
        z, parts = O.layer_forward(x, p, seq_len=seq, n_heads=h, causal=True, eps=1e-2, return_parts=True)
        assert np.max(np.abs((z - parts["y"]) - ref)) > 1e-3
        return
    elif mutation == "ln_no_eps":
        orig_ln = O.layer_norm
        monkeypatch.setattr(O, "layer_norm", lambda x_, g, b, eps: orig_ln(x_, g, b, 0.0))
    got = O.layer_forward(x, p, seq_len=seq, n_heads=h, causal=True, eps=1e-2)
    assert np.max(np.abs(got - ref)) > 1e-6, mutation


def test_stack4_32k_golden_file_is_well_formed():
    """The stored oracle rows of the 4-layer, 32768-token stack: the sampled rows the
    generator draws, one finite d-wide output row each, and an input digest."""
    from blockwise_attn_ffn_amd import synth
    w = synth.WORKLOADS["stack4_32k"]
    g = np.load(os.path.join(os.path.dirname(__file__), "golden", "stack4_32k_rows.npz"))
    assert np.array_equal(g["rows"], synth.sample_rows(w, w.sample_rows, seed=0))
    assert g["z"].shape == (w.sample_rows, w.d_model) and g["z"].dtype == np.float64
    assert np.isfinite(g["z"]).all()
    assert len(str(g["input_sha256"])) == 64


# --------------------------------------------------------------------------
# Saved softmax statistics: lse = m + log l per row and head
# --------------------------------------------------------------------------

def brute_force_lse(q, k, n_heads, causal):
    """Explicit loops, math.exp and math.log of the plain sum (no maximum taken:
    for the small scores used here)."""
    nq, d = q.shape
    dk = d // n_heads
    out = np.zeros((n_heads, nq))
    for h in range(n_heads):
        for i in range(nq):
            keys = range(i + 1) if causal else range(k.shape[0])
            tot = math.fsum(math.exp(sum(q[i, h * dk + c] * k[j, h * dk + c] for c in range(dk))
                                     / math.sqrt(dk)) for j in keys)
            out[h, i] = math.log(tot)
    return out


def _lse_pins(fn):
    """True iff fn(q, k, n_heads, causal) passes every pin below."""
    rng = np.random.default_rng(21)
    for causal in (False, True):
        q, k = rng.standard_normal((7, 8)), rng.standard_normal((7, 8))
        if not np.allclose(fn(q, k, 2, causal), brute_force_lse(q, k, 2, causal), atol=1e-12, rtol=0):
            return False
        z = np.zeros((5, 8))
        want = np.log(np.arange(1, 6)) if causal else np.full(5, math.log(5))
        if not np.allclose(fn(z, rng.standard_normal((5, 8)), 2, causal), want[None, :], atol=1e-12, rtol=0):
            return False
    # two keys tie at a huge score: lse = that score + log 2, exactly representable path
    q = np.zeros((1, 4)); q[0, 0] = 1.0
    k = np.zeros((3, 4)); k[0, 0] = k[1, 0] = 1000.0 * 2.0; k[2, 0] = -1000.0
    with np.errstate(over="ignore", invalid="ignore"):
        got = fn(q, k, 1, False)
    return bool(np.isfinite(got).all() and abs(got[0, 0] - (1000.0 + math.log(2.0))) < 1e-9)


def test_lse_pins_hold_for_the_oracle():
    assert _lse_pins(oracle.attention_lse_sequence)


@pytest.mark.parametrize("causal", [False, True])
def test_lse_recovers_the_attention_output(causal):
    """exp(S - lse) V, with S the scaled scores, is the oracle's attention output:
    the saved statistic is the normaliser its softmax used."""
    rng = np.random.default_rng(22 + causal)
    n, d, h = 11, 16, 2
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    lse = oracle.attention_lse_sequence(q, k, h, causal)
    want = oracle.attention_sequence(q, k, v, h, causal)
    dk = d // h
    for hh in range(h):
        c = slice(hh * dk, (hh + 1) * dk)
        s = q[:, c] @ k[:, c].T / math.sqrt(dk)
        if causal:
            s = np.where(np.arange(n)[None, :] > np.arange(n)[:, None], -np.inf, s)
        assert np.max(np.abs(np.exp(s - lse[hh][:, None]) @ v[:, c] - want[:, c])) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_layer_lse_rows_equal_full(causal):
    rng = np.random.default_rng(23 + causal)
    n, b, d, h = 20, 2, 16, 2
    p = rand_layer(rng, d, 4 * d)
    x = rng.standard_normal((b * n, d))
    full = oracle.layer_lse(x, p, seq_len=n, n_heads=h, causal=causal)
    rows = np.array([0, 3, 19, 20, 31, 39])
    got = oracle.layer_lse_rows(x, p, rows, seq_len=n, n_heads=h, causal=causal, row_chunk=7)
    want = np.stack([full[r // n, :, r % n] for r in rows])
    assert np.max(np.abs(got - want)) < 1e-12


def test_lse_pins_catch_planted_mistakes():
    """Each plausible slip in the statistic fails at least one pin."""
    base = oracle.attention_lse_sequence

    def no_scale(q, k, nh, causal):
        return base(q * math.sqrt(q.shape[1] // nh), k, nh, causal)

    def log2(q, k, nh, causal):
        return base(q, k, nh, causal) / math.log(2.0)

    def max_dropped(q, k, nh, causal):
        dk = q.shape[1] // nh
        out = np.empty((nh, q.shape[0]))
        for hh in range(nh):
            c = slice(hh * dk, (hh + 1) * dk)
            s = q[:, c] @ k[:, c].T / math.sqrt(dk)
            if causal:
                s = np.where(np.arange(k.shape[0])[None, :] > np.arange(q.shape[0])[:, None], -np.inf, s)
            out[hh] = np.log(np.exp(s).sum(axis=1))
        return out

    def causal_off_by_one(q, k, nh, causal):
        if not causal:
            return base(q, k, nh, causal)
        return base(q, k, nh, False) if q.shape[0] < 2 else np.concatenate(
            [base(q[:1], k[:1], nh, False), base(q[1:], k, nh, True, q_pos=np.arange(q.shape[0] - 1))],
            axis=1)

    for planted in (no_scale, log2, max_dropped, causal_off_by_one):
        assert not _lse_pins(planted), planted.__name__


# --------------------------------------------------------------------------
# Attention backward (the part of the backward pass the saved statistics serve)
# --------------------------------------------------------------------------

def _attn_loss(q, k, v, g, h, causal):
    return float((oracle.attention_sequence(q, k, v, h, causal) * g).sum())


def _bwd_pins(fn):
    """True iff fn(q, k, v, do, n_heads, causal) -> (dq, dk, dv) passes the pins."""
    rng = np.random.default_rng(31)
    for causal in (False, True):
        n, d, h = 6, 8, 2
        q, k, v, g = (rng.standard_normal((n, d)) for _ in range(4))
        dq, dk, dv = fn(q, k, v, g, h, causal)
        eps = 1e-6
        for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            fd = np.empty_like(x)
            for idx in np.ndindex(*x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += eps
                xm[idx] -= eps
                args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
                args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
                fd[idx] = (_attn_loss(*args_p, g, h, causal) - _attn_loss(*args_m, g, h, causal)) / (2 * eps)
            if np.max(np.abs(fd - grad)) > 1e-7:
                return False
    return True


def test_attention_backward_pins_hold_for_the_oracle():
    assert _bwd_pins(oracle.attention_backward_sequence)


@pytest.mark.parametrize("causal", [False, True])
def test_attention_backward_matches_torch_autograd(causal):
    rng = np.random.default_rng(32 + causal)
    n, d, h = 13, 16, 2
    q, k, v, g = (rng.standard_normal((n, d)) for _ in range(4))
    tq, tk, tv = (torch.from_numpy(a.copy()).requires_grad_(True) for a in (q, k, v))
    split = lambda t: t.view(n, h, d // h).transpose(0, 1)  # noqa: E731
    a = F.scaled_dot_product_attention(split(tq)[None], split(tk)[None], split(tv)[None], is_causal=causal)
    (a[0].transpose(0, 1).reshape(n, d) * torch.from_numpy(g)).sum().backward()
    dq, dk, dv = oracle.attention_backward_sequence(q, k, v, g, h, causal)
    for got, t in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.max(np.abs(got - t.grad.numpy())) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_attention_backward_invariants(causal):
    """Shifting every key by one vector leaves each row's softmax unchanged, so the
    gradients of a head's keys sum to zero; rowsum(P * dP) = rowsum(dO * A)."""
    rng = np.random.default_rng(34 + causal)
    n, d, h = 12, 16, 2
    q, k, v, g = (rng.standard_normal((n, d)) for _ in range(4))
    _, dk, _ = oracle.attention_backward_sequence(q, k, v, g, h, causal)
    assert np.max(np.abs(dk.sum(axis=0))) < 1e-12
    a = oracle.attention_sequence(q, k, v, h, causal)
    dkh = d // h
    for hh in range(h):
        c = slice(hh * dkh, (hh + 1) * dkh)
        s = q[:, c] @ k[:, c].T / math.sqrt(dkh)
        if causal:
            s = np.where(np.arange(n)[None, :] > np.arange(n)[:, None], -np.inf, s)
        pm = oracle.softmax_rows(s)
        assert np.max(np.abs((pm * (g[:, c] @ v[:, c].T)).sum(axis=1) - (g[:, c] * a[:, c]).sum(axis=1))) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_attention_backward_dq_rows_equal_full(causal):
    rng = np.random.default_rng(36 + causal)
    n, d, h = 17, 16, 2
    q, k, v, g = (rng.standard_normal((n, d)) for _ in range(4))
    dq, _, _ = oracle.attention_backward_sequence(q, k, v, g, h, causal)
    rows = np.array([0, 1, 8, 16])
    got = oracle.attention_backward_dq_rows(q, k, v, g, h, causal, rows)
    assert np.max(np.abs(got - dq[rows])) < 1e-12


def test_attention_backward_pins_catch_planted_mistakes():
    base = oracle.attention_backward_sequence

    def no_rowsum_term(q, k, v, g, h, causal):
        # dS = P * dP (the Jacobian's second term dropped)
        dq, dk, dv = base(q, k, v, g, h, causal)
        n, d = q.shape
        dkh = d // h
        dq2, dk2 = np.empty_like(dq), np.empty_like(dk)
        for hh in range(h):
            c = slice(hh * dkh, (hh + 1) * dkh)
            s = q[:, c] @ k[:, c].T / math.sqrt(dkh)
            if causal:
                s = np.where(np.arange(n)[None, :] > np.arange(n)[:, None], -np.inf, s)
            pm = oracle.softmax_rows(s)
            ds = pm * (g[:, c] @ v[:, c].T)
            dq2[:, c] = ds @ k[:, c] / math.sqrt(dkh)
            dk2[:, c] = ds.T @ q[:, c] / math.sqrt(dkh)
        return dq2, dk2, dv

    def no_scale_on_dq(q, k, v, g, h, causal):
        dq, dk, dv = base(q, k, v, g, h, causal)
        return dq * math.sqrt(q.shape[1] // h), dk, dv

    def p_not_transposed(q, k, v, g, h, causal):
        dq, dk, dv = base(q, k, v, g, h, causal)
        n, d = q.shape
        dkh = d // h
        dv2 = np.empty_like(dv)
        for hh in range(h):
            c = slice(hh * dkh, (hh + 1) * dkh)
            s = q[:, c] @ k[:, c].T / math.sqrt(dkh)
            if causal:
                s = np.where(np.arange(n)[None, :] > np.arange(n)[:, None], -np.inf, s)
            dv2[:, c] = oracle.softmax_rows(s) @ g[:, c]
        return dq, dk, dv2

    for planted in (no_rowsum_term, no_scale_on_dq, p_not_transposed):
        assert not _bwd_pins(planted), planted.__name__


@pytest.mark.parametrize("causal", [False, True])
def test_attention_backward_kv_rows_equal_full(causal):
    """dK, dV at chosen keys equal the full backward's, with dO dense and with dO
    zero on most rows (those queries are then skipped)."""
    rng = np.random.default_rng(38 + causal)
    n, d, h = 19, 16, 2
    q, k, v, g = (rng.standard_normal((n, d)) for _ in range(4))
    rows = np.array([0, 3, 9, 17, 18])
    for sparse in (False, True):
        gg = g.copy()
        if sparse:
            gg[np.setdiff1d(np.arange(n), [2, 9, 18])] = 0.0
        _, dk, dv = oracle.attention_backward_sequence(q, k, v, gg, h, causal)
        got_k, got_v = oracle.attention_backward_kv_rows(q, k, v, gg, h, causal, rows)
        assert np.max(np.abs(got_k - dk[rows])) < 1e-12
        assert np.max(np.abs(got_v - dv[rows])) < 1e-12
        assert np.max(np.abs(got_v[-1])) > 0          # key 18 is seen by query 18 (live)


# --------------------------------------------------------------------------
# Window and chunked-streaming masks (transformer-cost page, Section 5)
# --------------------------------------------------------------------------

def _mask_pins(attn):
    """True iff attn(q, k, v, h, causal, window=, chunk=) -> [n, d] passes the mask pins."""
    rng = np.random.default_rng(41)
    n, d, h = 13, 8, 2
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    causal = oracle.attention_sequence(q, k, v, h, True)
    full = oracle.attention_sequence(q, k, v, h, False)
    checks = [
        np.max(np.abs(attn(q, k, v, h, True, window=1) - v)) < 1e-12,        # a token sees only itself
        np.max(np.abs(attn(q, k, v, h, True, window=n) - causal)) < 1e-12,   # full length: causal
        np.max(np.abs(attn(q, k, v, h, True, window=n + 5) - causal)) < 1e-12,
        np.max(np.abs(attn(q, k, v, h, True, chunk=1) - causal)) < 1e-12,    # chunk 1: causal
        np.max(np.abs(attn(q, k, v, h, True, chunk=n) - full)) < 1e-12,      # whole length: no mask
    ]
    # the page's example: chunk size 4, token 9 reads tokens 10 and 11 but not 12
    for key, seen in ((10, True), (11, True), (12, False), (8, True)):
        k2 = k.copy()
        k2[key] += 1.0
        moved = np.max(np.abs(attn(q, k2, v, h, True, chunk=4)[9] - attn(q, k, v, h, True, chunk=4)[9])) > 1e-9
        checks.append(moved == seen)
    # window w: row i reads key i - w + 1 and not key i - w
    w, i = 4, 10
    for key, seen in ((i - w + 1, True), (i - w, False), (i, True)):
        k2 = k.copy()
        k2[key] += 1.0
        moved = np.max(np.abs(attn(q, k2, v, h, True, window=w)[i] - attn(q, k, v, h, True, window=w)[i])) > 1e-9
        checks.append(moved == seen)
    return all(checks)


def test_mask_pins_hold_for_the_oracle():
    assert _mask_pins(oracle.attention_sequence)


def test_mask_pins_catch_planted_mistakes():
    base = oracle.attention_sequence

    def shifted_window(q, k, v, h, causal, window=0, chunk=0):
        return base(q, k, v, h, causal, window=window + 1 if window else 0, chunk=chunk)

    def chunk_as_causal_within(q, k, v, h, causal, window=0, chunk=0):
        # keys of the own chunk only up to the query (a plain causal mask inside the chunk)
        return base(q, k, v, h, causal, window=window) if chunk else base(q, k, v, h, causal, window=window)

    def chunk_next_chunk(q, k, v, h, causal, window=0, chunk=0):
        # one chunk too many: the next chunk visible as well
        return base(q, k, v, h, causal, window=window, chunk=2 * chunk) if chunk else base(
            q, k, v, h, causal, window=window)

    for planted in (shifted_window, chunk_as_causal_within, chunk_next_chunk):
        assert not _mask_pins(planted), planted.__name__


@pytest.mark.parametrize("mask", [dict(window=3), dict(window=17), dict(chunk=5), dict(chunk=16)])
def test_masked_attention_matches_torch_sdpa_with_explicit_mask(mask):
    """The masked softmax attention itself against torch's float64 SDPA given the same
    boolean mask (built here by a loop over the page's rule)."""
    rng = np.random.default_rng(43)
    n, d, h = 37, 16, 2
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    allowed = np.zeros((n, n), dtype=bool)
    for i in range(n):
        if "window" in mask:
            allowed[i, max(0, i - mask["window"] + 1):i + 1] = True
        else:
            allowed[i, :min(n, (i // mask["chunk"] + 1) * mask["chunk"])] = True
    split = lambda a: torch.from_numpy(a.copy()).view(n, h, d // h).transpose(0, 1)[None]  # noqa: E731
    ref = F.scaled_dot_product_attention(split(q), split(k), split(v),
                                         attn_mask=torch.from_numpy(allowed))
    ref = ref[0].transpose(0, 1).reshape(n, d).numpy()
    got = oracle.attention_sequence(q, k, v, h, True, **mask)
    assert np.max(np.abs(got - ref)) < 1e-12


@pytest.mark.parametrize("mask", [dict(window=5), dict(window=40), dict(chunk=7), dict(chunk=32)])
def test_blockwise_loop_with_masks_equals_unfused(mask):
    rng = np.random.default_rng(45)
    seq, d, h = 45, 16, 2
    x = rng.standard_normal((2 * seq, d))
    p = rand_layer(rng, d, 64, std=0.3)
    ref = oracle.layer_forward(x, p, seq_len=seq, n_heads=h, causal=True, **mask)
    for bq, bkv in ((8, 8), (16, 4), (4, 16)):
        got = oracle.blockwise_layer_forward(x, p, seq_len=seq, n_heads=h, causal=True, block_q=bq,
                                             block_kv=bkv, **mask)
        assert np.max(np.abs(got - ref)) < 1e-10, (bq, bkv)


@pytest.mark.parametrize("mask", [dict(window=6), dict(chunk=8)])
def test_masked_rows_and_lse_equal_full(mask):
    rng = np.random.default_rng(47)
    seq, d, h = 40, 16, 2
    x = rng.standard_normal((2 * seq, d))
    p = rand_layer(rng, d, 64, std=0.3)
    rows = np.array([0, 5, 17, 39, 40, 47, 79])
    full = oracle.layer_forward(x, p, seq_len=seq, n_heads=h, causal=True, **mask)
    got = oracle.layer_forward_rows(x, p, rows, seq_len=seq, n_heads=h, causal=True, **mask)
    assert np.max(np.abs(got - full[rows])) < 1e-12
    lse = oracle.layer_lse(x, p, seq_len=seq, n_heads=h, causal=True, **mask)
    lse_r = oracle.layer_lse_rows(x, p, rows, seq_len=seq, n_heads=h, causal=True, **mask)
    assert np.max(np.abs(lse_r - lse[rows // seq, :, rows % seq])) < 1e-12


def test_window_one_lse_is_the_diagonal_score():
    rng = np.random.default_rng(49)
    n, d, h = 9, 8, 2
    q, k = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    lse = oracle.attention_lse_sequence(q, k, h, True, window=1)
    for hh in range(h):
        c = slice(hh * 4, hh * 4 + 4)
        assert np.max(np.abs(lse[hh] - (q[:, c] * k[:, c]).sum(1) / 2.0)) < 1e-12


# --------------------------------------------------------------------------
# Grouped-query attention (transformer-cost page, MQA and GQA)
# --------------------------------------------------------------------------

def _gqa_pins(attn):
    """True iff attn(q, k, v, n_heads, causal) with K, V of g heads passes the pins."""
    rng = np.random.default_rng(51)
    n, h, dk = 11, 8, 4
    ok = []
    for g in (1, 2, 4):
        q = rng.standard_normal((n, h * dk))
        k, v = rng.standard_normal((n, g * dk)), rng.standard_normal((n, g * dk))
        for causal in (False, True):
            # torch's SDPA with enable_gqa (float64)
            sq = torch.from_numpy(q.copy()).view(n, h, dk).transpose(0, 1)[None]
            sk = torch.from_numpy(k.copy()).view(n, g, dk).transpose(0, 1)[None]
            sv = torch.from_numpy(v.copy()).view(n, g, dk).transpose(0, 1)[None]
            ref = F.scaled_dot_product_attention(sq, sk, sv, is_causal=causal, enable_gqa=True)
            ref = ref[0].transpose(0, 1).reshape(n, h * dk).numpy()
            ok.append(np.max(np.abs(attn(q, k, v, h, causal) - ref)) < 1e-12)
            # the page's construction: each key/value head repeated for its group
            rep = lambda a: np.repeat(a.reshape(n, g, dk), h // g, axis=1).reshape(n, h * dk)  # noqa: E731
            ok.append(np.max(np.abs(attn(q, k, v, h, causal) - attn(q, rep(k), rep(v), h, causal))) < 1e-12)
    return all(ok)


def test_gqa_pins_hold_for_the_oracle():
    assert _gqa_pins(lambda q, k, v, h, c: oracle.attention_sequence(q, k, v, h, c))


def test_gqa_pins_catch_planted_mistake():
    def modulo_mapping(q, k, v, h, causal):
        # query head h reads key/value head h % g instead of h // (h / g)
        dk = q.shape[1] // h
        g = k.shape[1] // dk
        perm = np.concatenate([np.arange((hh % g) * dk, (hh % g + 1) * dk) for hh in range(h)])
        return oracle.attention_sequence(q, k[:, perm], v[:, perm], h, causal)
    assert not _gqa_pins(modulo_mapping)


def test_mqa_every_head_reads_the_same_keys():
    rng = np.random.default_rng(53)
    n, h, dk = 9, 4, 8
    q = rng.standard_normal((n, dk))
    q4 = np.tile(q, (1, h))                          # the same query in every head
    k, v = rng.standard_normal((n, dk)), rng.standard_normal((n, dk))
    out = oracle.attention_sequence(q4, k, v, h, True)
    one = oracle.attention_sequence(q, k, v, 1, True)
    for hh in range(h):
        assert np.max(np.abs(out[:, hh * dk:(hh + 1) * dk] - one)) < 1e-12


@pytest.mark.parametrize("g,mask", [(1, {}), (2, dict(window=6)), (2, dict(chunk=8))])
def test_gqa_layer_blockwise_and_rows_equal_unfused(g, mask):
    rng = np.random.default_rng(55)
    seq, d, h = 37, 16, 4
    x = rng.standard_normal((2 * seq, d))
    p = rand_layer(rng, d, 64, std=0.3)
    dkv = g * (d // h)
    p["w_k"] = p["w_k"][:, :dkv].copy()
    p["w_v"] = p["w_v"][:, :dkv].copy()
    ref = oracle.layer_forward(x, p, seq_len=seq, n_heads=h, causal=True, **mask)
    got = oracle.blockwise_layer_forward(x, p, seq_len=seq, n_heads=h, causal=True, block_q=8,
                                         block_kv=16, **mask)
    assert np.max(np.abs(got - ref)) < 1e-10
    rows = np.array([0, 9, 36, 37, 73])
    assert np.max(np.abs(oracle.layer_forward_rows(x, p, rows, seq_len=seq, n_heads=h, causal=True,
                                                   **mask) - ref[rows])) < 1e-12
    lse = oracle.layer_lse(x, p, seq_len=seq, n_heads=h, causal=True, **mask)
    lse_r = oracle.layer_lse_rows(x, p, rows, seq_len=seq, n_heads=h, causal=True, **mask)
    assert np.max(np.abs(lse_r - lse[rows // seq, :, rows % seq])) < 1e-12



def _bwd_pins_general(fn, mask, g):
    """Central finite differences of sum(A * G) through attention_sequence (pinned on
    its own) with a mask and g key/value heads."""
    rng = np.random.default_rng(61)
    n, h, dkh = 7, 4, 2
    q = rng.standard_normal((n, h * dkh))
    k, v = rng.standard_normal((n, g * dkh)), rng.standard_normal((n, g * dkh))
    gg = rng.standard_normal((n, h * dkh))
    loss = lambda q_, k_, v_: float((oracle.attention_sequence(q_, k_, v_, h, True, **mask) * gg).sum())  # noqa: E731
    dq, dk, dv = fn(q, k, v, gg, h, True, **mask)
    eps = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.empty_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            a_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            a_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd[idx] = (loss(*a_p) - loss(*a_m)) / (2 * eps)
        if np.max(np.abs(fd - grad)) > 1e-7:
            return False
    return True


@pytest.mark.parametrize("mask,g", [(dict(window=3), 4), (dict(chunk=3), 4), ({}, 2), ({}, 1),
                                    (dict(window=2), 2), (dict(chunk=2), 1)])
def test_backward_with_masks_and_grouped_heads_pinned_by_finite_differences(mask, g):
    assert _bwd_pins_general(oracle.attention_backward_sequence, mask, g)


def test_backward_general_pins_catch_planted_mistakes():
    base = oracle.attention_backward_sequence

    def grouped_dk_not_summed(q, k, v, do, h, causal, **mask):
        # dK of a key/value head taken from its first query head only
        dq, dk, dv = base(q, k, v, do, h, causal, **mask)
        g = k.shape[1] // (q.shape[1] // h)
        dkh = q.shape[1] // h
        first = np.concatenate([q[:, (hh * (h // g)) * dkh:(hh * (h // g) + 1) * dkh] for hh in range(g)], axis=1)
        _, dk1, _ = base(first, k, v, do[:, :first.shape[1]], g, causal, **mask)
        return dq, dk1, dv

    def mask_ignored(q, k, v, do, h, causal, **mask):
        return base(q, k, v, do, h, causal)

    assert not _bwd_pins_general(grouped_dk_not_summed, {}, 2)
    assert not _bwd_pins_general(mask_ignored, dict(window=3), 4)


@pytest.mark.parametrize("mask,g", [(dict(window=5), 2), (dict(chunk=4), 1), ({}, 2)])
def test_backward_rows_forms_equal_full_with_masks_and_groups(mask, g):
    rng = np.random.default_rng(63)
    n, h, dkh = 21, 4, 4
    q = rng.standard_normal((n, h * dkh))
    k, v = rng.standard_normal((n, g * dkh)), rng.standard_normal((n, g * dkh))
    gg = rng.standard_normal((n, h * dkh))
    gg[np.setdiff1d(np.arange(n), [3, 11, 20])] = 0.0
    dq, dk, dv = oracle.attention_backward_sequence(q, k, v, gg, h, True, **mask)
    rows = np.array([0, 3, 11, 19, 20])
    assert np.max(np.abs(oracle.attention_backward_dq_rows(q, k, v, gg, h, True, rows, **mask) - dq[rows])) < 1e-12
    rk, rv = oracle.attention_backward_kv_rows(q, k, v, gg, h, True, rows, **mask)
    assert np.max(np.abs(rk - dk[rows])) < 1e-12 and np.max(np.abs(rv - dv[rows])) < 1e-12


# --------------------------------------------------------------------------
# The layer's saved statistic (layer_lse, layer_lse_rows) against torch
# --------------------------------------------------------------------------

def torch_layer_lse(x, p, seq_len, n_heads, causal, eps=1e-5, window=0, chunk=0):
    """[B, n_heads, seq_len] from torch CPU float64 ops alone: F.layer_norm with the
    first LN's parameters, Q = LN1(x) W_Q, K = LN1(x) W_K, scaled scores per head with
    the mask built from positions here, then torch.logsumexp over the keys."""
    t = {k: torch.from_numpy(np.asarray(v, np.float64)) for k, v in p.items()}
    xt = torch.from_numpy(np.asarray(x, np.float64))
    rows, d = xt.shape
    dk = d // n_heads
    x1 = F.layer_norm(xt, (d,), t["ln1_g"], t["ln1_b"], eps)
    q, k = x1 @ t["w_q"], x1 @ t["w_k"]
    g = k.shape[1] // dk
    pos = torch.arange(seq_len)
    allowed = torch.ones(seq_len, seq_len, dtype=torch.bool)
    if causal:
        allowed = pos[None, :] <= pos[:, None]
        if window:
            allowed &= pos[None, :] > pos[:, None] - window
        if chunk:
            allowed = (pos[None, :] // chunk) <= (pos[:, None] // chunk)
    out = torch.empty(rows // seq_len, n_heads, seq_len, dtype=torch.float64)
    for b in range(rows // seq_len):
        sl = slice(b * seq_len, (b + 1) * seq_len)
        for h in range(n_heads):
            kh = h // (n_heads // g)
            s = q[sl, h * dk:(h + 1) * dk] @ k[sl, kh * dk:(kh + 1) * dk].T / math.sqrt(dk)
            out[b, h] = torch.logsumexp(s.masked_fill(~allowed, -math.inf), dim=1)
    return out.numpy()


def torch_attention_heads(x, p, seq_len, n_heads, causal, eps=1e-5):
    """Per-sequence attention output [rows, d] from torch's layer_norm, matmuls and
    scaled_dot_product_attention (float64), with the V it used."""
    t = {k: torch.from_numpy(np.asarray(v, np.float64)) for k, v in p.items()}
    xt = torch.from_numpy(np.asarray(x, np.float64))
    rows, d = xt.shape
    dk = d // n_heads
    x1 = F.layer_norm(xt, (d,), t["ln1_g"], t["ln1_b"], eps)
    split = lambda a: a.view(rows // seq_len, seq_len, n_heads, dk).transpose(1, 2)  # noqa: E731
    q, k, v = x1 @ t["w_q"], x1 @ t["w_k"], x1 @ t["w_v"]
    a = F.scaled_dot_product_attention(split(q), split(k), split(v), is_causal=causal)
    return a.transpose(1, 2).reshape(rows, d).numpy(), q.numpy(), k.numpy(), v.numpy()


def _layer_lse_pins(full_fn, rows_fn):
    """True iff full_fn (layer_lse's signature) and rows_fn (layer_lse_rows') pass:
    torch's logsumexp of the masked scores built from torch's LN and matmuls (random
    LN gains and biases that differ between the two LNs), and the recovery of torch's
    SDPA output as exp(S_h - lse_h) V_h for every head."""
    rng = np.random.default_rng(71)
    seq, b, d, h = 13, 2, 16, 2
    dk = d // h
    x = rng.standard_normal((b * seq, d)) * 1.5 + 0.3
    p = rand_layer(rng, d, 4 * d, std=0.4)
    rows = np.array([0, 4, 12, 13, 20, 25])
    for causal, mask in ((False, {}), (True, {}), (True, dict(window=4)), (True, dict(chunk=5))):
        want = torch_layer_lse(x, p, seq, h, causal, **mask)
        got = full_fn(x, p, seq_len=seq, n_heads=h, causal=causal, **mask)
        if got.shape != want.shape or np.max(np.abs(got - want)) > 1e-12:
            return False
        got_r = rows_fn(x, p, rows, seq_len=seq, n_heads=h, causal=causal, **mask)
        if np.max(np.abs(got_r - want[rows // seq, :, rows % seq])) > 1e-12:
            return False
    for causal in (False, True):
        a, q, k, v = torch_attention_heads(x, p, seq, h, causal)
        lse = full_fn(x, p, seq_len=seq, n_heads=h, causal=causal)
        for bb in range(b):
            sl = slice(bb * seq, (bb + 1) * seq)
            for hh in range(h):
                c = slice(hh * dk, (hh + 1) * dk)
                s = q[sl, c] @ k[sl, c].T / math.sqrt(dk)
                if causal:
                    s = np.where(np.arange(seq)[None, :] > np.arange(seq)[:, None], -np.inf, s)
                if np.max(np.abs(np.exp(s - lse[bb, hh][:, None]) @ v[sl, c] - a[sl, c])) > 1e-12:
                    return False
    return True


def test_layer_lse_pins_hold_for_the_oracle():
    assert _layer_lse_pins(oracle.layer_lse, oracle.layer_lse_rows)


def test_layer_lse_pins_catch_planted_mistakes(monkeypatch):
    """Slips that a self-comparison (rows == full) cannot see: the FFN's LN parameters
    used for the attention's LN, W_K used for the queries, LN left out."""
    def ln2_for_ln1(fn):
        return lambda x, p, *a, **kw: fn(x, dict(p, ln1_g=p["ln2_g"], ln1_b=p["ln2_b"]), *a, **kw)

    def wk_for_q(fn):
        return lambda x, p, *a, **kw: fn(x, dict(p, w_q=p["w_k"]), *a, **kw)

    for planted in (ln2_for_ln1, wk_for_q):
        assert not _layer_lse_pins(planted(oracle.layer_lse), oracle.layer_lse_rows), planted.__name__
        assert not _layer_lse_pins(oracle.layer_lse, planted(oracle.layer_lse_rows)), planted.__name__
    with monkeypatch.context() as mp:
        mp.setattr(O, "layer_norm", lambda x_, g, b, eps: np.asarray(x_, np.float64))
        assert not _layer_lse_pins(O.layer_lse, O.layer_lse_rows), "ln_dropped"


def test_summaries_merge_in_any_grouping_to_the_full_softmax():
    """Cut a score row at random points, summarise each piece, merge the pieces in a
    random order and grouping: o / l is scipy's softmax-weighted mean, l its
    normaliser at the row maximum; an empty piece changes nothing."""
    rng = np.random.default_rng(73)
    for trial in range(20):
        n = int(rng.integers(1, 40))
        s = rng.standard_normal(n) * 3
        v = rng.standard_normal((n, 3))
        cuts = np.sort(rng.choice(np.arange(1, n), size=min(n - 1, int(rng.integers(0, 6))),
                                  replace=False)) if n > 1 else np.array([], int)
        pieces = [O.softmax_summary(a, b) for a, b in zip(np.split(s, cuts), np.split(v, cuts))]
        pieces.append(O.softmax_summary(np.full(2, -np.inf), np.ones((2, 3))))   # empty set
        order = rng.permutation(len(pieces))
        acc = pieces[order[0]]
        for i in order[1:]:
            acc = O.merge_summaries(pieces[i], acc) if i % 2 else O.merge_summaries(acc, pieces[i])
        m, l, o = acc
        assert m == s.max()
        assert abs(l - np.exp(s - s.max()).sum()) < 1e-12 * n
        assert np.max(np.abs(o / l - scipy.special.softmax(s) @ v)) < 1e-12


def test_fused_pin_catches_a_merge_without_rescaling(monkeypatch):
    """A merge that adds the two sums without moving them to the common maximum
    breaks blockwise == unfused."""
    def bad(a, b):
        (ma, la, oa), (mb, lb, ob) = a, b
        return np.maximum(ma, mb), la + lb, oa + ob
    monkeypatch.setattr(O, "merge_summaries", bad)
    rng = np.random.default_rng(74)
    seq, d, h = 32, 16, 2
    x = rng.standard_normal((seq, d))
    p = rand_layer(rng, d, 64, std=0.4)
    ref = O.layer_forward(x, p, seq_len=seq, n_heads=h, causal=True)
    got = O.blockwise_layer_forward(x, p, seq_len=seq, n_heads=h, causal=True, block_q=16, block_kv=8)
    assert O.rel_fro_err(got, ref) > 1e-6


# --------------------------------------------------------------------------
# The layer backward (block-recompute backward: the plain definition it must match)
# --------------------------------------------------------------------------

_GRAD_KEYS = ("dw_q", "dw_k", "dw_v", "dw_o", "dw_1", "dw_2", "dln1_g", "dln1_b", "dln2_g", "dln2_b")
_PARAM_OF = {"dw_q": "w_q", "dw_k": "w_k", "dw_v": "w_v", "dw_o": "w_o", "dw_1": "w_1", "dw_2": "w_2",
             "dln1_g": "ln1_g", "dln1_b": "ln1_b", "dln2_g": "ln2_g", "dln2_b": "ln2_b"}


def torch_layer_grads(x, p, dz, seq_len, n_heads, causal, eps=1e-5):
    """dL/dX and dL/dparam for L = sum(Z * dz), Z from the torch-built layer
    (F.layer_norm, matmuls, scaled_dot_product_attention, gelu), by torch float64
    autograd."""
    t = {k: torch.tensor(np.asarray(v, np.float64), requires_grad=True) for k, v in p.items()}
    xt = torch.tensor(np.asarray(x, np.float64), requires_grad=True)
    rows, d = xt.shape
    dk = d // n_heads
    x1 = F.layer_norm(xt, (d,), t["ln1_g"], t["ln1_b"], eps)
    split = lambda a: a.view(rows // seq_len, seq_len, n_heads, dk).transpose(1, 2)  # noqa: E731
    a = F.scaled_dot_product_attention(split(x1 @ t["w_q"]), split(x1 @ t["w_k"]),
                                       split(x1 @ t["w_v"]), is_causal=causal)
    a = a.transpose(1, 2).reshape(rows, d)
    y = xt + a @ t["w_o"]
    h = F.gelu(F.layer_norm(y, (d,), t["ln2_g"], t["ln2_b"], eps) @ t["w_1"], approximate="tanh")
    z = y + h @ t["w_2"]
    (z * torch.from_numpy(np.asarray(dz, np.float64))).sum().backward()
    out = {"dx": xt.grad.numpy()}
    for gk, pk in _PARAM_OF.items():
        out[gk] = t[pk].grad.numpy()
    return out


def _layer_bwd_pins(fn):
    """True iff fn (layer_backward's signature) agrees with torch autograd (every
    gradient, causal and not, random LN parameters) and with central finite
    differences of L = sum(Z * dz) on sampled entries of X and of every parameter."""
    rng = np.random.default_rng(81)
    seq, b, d, h = 6, 2, 8, 2
    for causal in (False, True):
        x = rng.standard_normal((b * seq, d))
        p = rand_layer(rng, d, 4 * d, std=0.5)
        dz = rng.standard_normal((b * seq, d))
        got = fn(x, p, dz, seq_len=seq, n_heads=h, causal=causal)
        want = torch_layer_grads(x, p, dz, seq, h, causal)
        for key in ("dx",) + _GRAD_KEYS:
            if got[key].shape != want[key].shape or np.max(np.abs(got[key] - want[key])) > 1e-10:
                return False
    # finite differences on a few entries of each input (causal)
    x = rng.standard_normal((seq, d))
    p = rand_layer(rng, d, 4 * d, std=0.5)
    dz = rng.standard_normal((seq, d))
    got = fn(x, p, dz, seq_len=seq, n_heads=h, causal=True)
    loss = lambda xx, pp: float((oracle.layer_forward(xx, pp, seq_len=seq, n_heads=h, causal=True) * dz).sum())  # noqa: E731
    eps = 1e-6
    for key in ("dx",) + _GRAD_KEYS:
        base = x if key == "dx" else p[_PARAM_OF[key]]
        for _ in range(3):
            idx = tuple(int(rng.integers(0, n)) for n in base.shape)
            bp, bm = base.copy(), base.copy()
            bp[idx] += eps
            bm[idx] -= eps
            if key == "dx":
                fd = (loss(bp, p) - loss(bm, p)) / (2 * eps)
            else:
                fd = (loss(x, dict(p, **{_PARAM_OF[key]: bp})) - loss(x, dict(p, **{_PARAM_OF[key]: bm}))) / (2 * eps)
            if abs(fd - got[key][idx]) > 1e-6 * max(1.0, abs(fd)):
                return False
    return True


def test_layer_backward_pins_hold_for_the_oracle():
    assert _layer_bwd_pins(oracle.layer_backward)


def torch_layer_grads_masked(x, p, dz, seq_len, n_heads, eps=1e-5, window=0, chunk=0):
    """As torch_layer_grads (causal), with the attention written out from torch ops:
    per head the scaled scores, the mask built from positions here, torch.softmax and
    the values; query head h reads key/value head h // (n_heads / g), g from the
    width of W_K."""
    t = {k: torch.tensor(np.asarray(v, np.float64), requires_grad=True) for k, v in p.items()}
    xt = torch.tensor(np.asarray(x, np.float64), requires_grad=True)
    rows, d = xt.shape
    dk = d // n_heads
    x1 = F.layer_norm(xt, (d,), t["ln1_g"], t["ln1_b"], eps)
    q, k, v = x1 @ t["w_q"], x1 @ t["w_k"], x1 @ t["w_v"]
    g = k.shape[1] // dk
    pos = torch.arange(seq_len)
    allowed = pos[None, :] <= pos[:, None]
    if window:
        allowed &= pos[None, :] > pos[:, None] - window
    if chunk:
        allowed = (pos[None, :] // chunk) <= (pos[:, None] // chunk)
    seqs = []
    for b in range(rows // seq_len):
        sl = slice(b * seq_len, (b + 1) * seq_len)
        heads = []
        for h in range(n_heads):
            kh = h // (n_heads // g)
            s_ = q[sl, h * dk:(h + 1) * dk] @ k[sl, kh * dk:(kh + 1) * dk].T / math.sqrt(dk)
            heads.append(torch.softmax(s_.masked_fill(~allowed, -math.inf), dim=1) @ v[sl, kh * dk:(kh + 1) * dk])
        seqs.append(torch.cat(heads, dim=1))
    a = torch.cat(seqs, dim=0)
    y = xt + a @ t["w_o"]
    h_ = F.gelu(F.layer_norm(y, (d,), t["ln2_g"], t["ln2_b"], eps) @ t["w_1"], approximate="tanh")
    z = y + h_ @ t["w_2"]
    (z * torch.from_numpy(np.asarray(dz, np.float64))).sum().backward()
    out = {"dx": xt.grad.numpy()}
    for gk, pk in _PARAM_OF.items():
        out[gk] = t[pk].grad.numpy()
    return out


_MASK_CASES = [dict(window=3, g=2), dict(chunk=4, g=2), dict(g=1), dict(window=2, g=1)]


def _layer_bwd_mask_pins(fn):
    """True iff fn agrees with torch autograd (every gradient to 1e-10) on causal
    layers with a window, a chunked mask, one key/value head, and a window with one
    key/value head (2 query heads)."""
    rng = np.random.default_rng(97)
    seq, b, d, h = 8, 2, 8, 2
    dk = d // h
    for case in _MASK_CASES:
        x = rng.standard_normal((b * seq, d))
        p = rand_layer(rng, d, 4 * d, std=0.5)
        p["w_k"] = p["w_k"][:, :case["g"] * dk].copy()
        p["w_v"] = p["w_v"][:, :case["g"] * dk].copy()
        dz = rng.standard_normal((b * seq, d))
        kw = dict(window=case.get("window", 0), chunk=case.get("chunk", 0))
        got = fn(x, p, dz, seq_len=seq, n_heads=h, causal=True, **kw)
        want = torch_layer_grads_masked(x, p, dz, seq, h, **kw)
        for key in ("dx",) + _GRAD_KEYS:
            if got[key].shape != want[key].shape or np.max(np.abs(got[key] - want[key])) > 1e-10:
                return False
    return True


def test_layer_backward_masks_and_kv_heads_match_torch_autograd():
    assert _layer_bwd_mask_pins(oracle.layer_backward)


def test_layer_backward_mask_pins_catch_planted_mistakes(monkeypatch):
    """The attention backward run without the window / chunk, or a key/value head's
    gradients averaged over its query heads instead of summed, each fail."""
    real = O.attention_backward_sequence

    def unmasked(q, k, v, do, n_heads, causal, window=0, chunk=0):
        return real(q, k, v, do, n_heads, causal)

    def averaged(q, k, v, do, n_heads, causal, window=0, chunk=0):
        dq, dk, dv = real(q, k, v, do, n_heads, causal, window, chunk)
        r = n_heads * (q.shape[1] // n_heads) // k.shape[1]
        return dq, dk / r, dv / r

    for planted in (unmasked, averaged):
        with monkeypatch.context() as mp:
            mp.setattr(O, "attention_backward_sequence", planted)
            assert not _layer_bwd_mask_pins(O.layer_backward), planted.__name__


def test_layer_backward_pins_catch_planted_mistakes(monkeypatch):
    """Each slip fails a pin: the LN backward without its mean(g xh) term, GELU's
    derivative taken as the erf form's, W_1's gradient transposed into the wrong
    product, the first residual's gradient dropped."""
    def ln_no_second_term(x, gain, dy, eps):
        x = np.asarray(x, np.float64)
        xc = x - x.mean(axis=-1, keepdims=True)
        rstd = 1.0 / np.sqrt((xc * xc).mean(axis=-1, keepdims=True) + eps)
        g = dy * gain
        return rstd * (g - g.mean(axis=-1, keepdims=True)), (dy * xc * rstd).sum(0), dy.sum(0)

    def erf_derivative(u):
        return 0.5 * (1 + scipy.special.erf(u / math.sqrt(2))) + u * np.exp(-u * u / 2) / math.sqrt(2 * math.pi)

    with monkeypatch.context() as mp:
        mp.setattr(O, "layer_norm_backward", ln_no_second_term)
        assert not _layer_bwd_pins(O.layer_backward), "ln backward"
    with monkeypatch.context() as mp:
        mp.setattr(O, "gelu_tanh_derivative", erf_derivative)
        assert not _layer_bwd_pins(O.layer_backward), "gelu derivative"

    def w1_from_wrong_product(x, p, dz, **kw):
        g = O.layer_backward(x, p, dz, **kw)
        return dict(g, dw_1=g["dw_1"][::-1].copy())
    assert not _layer_bwd_pins(w1_from_wrong_product)

    def residual_dropped(x, p, dz, **kw):
        g = O.layer_backward(x, p, dz, **kw)
        return dict(g, dx=g["dx"] - np.asarray(dz, np.float64))
    assert not _layer_bwd_pins(residual_dropped)
