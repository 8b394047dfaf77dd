"""Plain CPU float64 oracle of the Blockwise Parallel Transformer (BPT) layer forward.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import or run this module. It shares no code with the HIP
library (no kernels, headers, helpers or constants), and imports nothing from it.

Sources (the pages this follows):
  [BPT]  "Blockwise Parallel Transformer — BPT" (aicassindra.com, transformer_math):
         sections "The fused blockwise algorithm", "The structural fact that makes
         fusion legal", "Pitfalls and misconceptions" (causal block skipping).
  [COST] "transformer-cost" (raminaeye.github.io): the FlashAttention paragraph and
         its two-tile running-sum example; the causal-mask and pitfalls table.

Notation follows [BPT]: X is the residual stream [N, d]; LN is a layer norm over
the feature axis; W_Q, W_K, W_V, W_O are [d, d]; W_1 is [d, d_ff], W_2 is
[d_ff, d]; every projection is y = x @ W (no linear biases); act is GELU with the
tanh approximation. Matrices here are in that orientation (in, out).

Readings of points the pages leave open (each also listed in the design notes):
  * LN: biased variance over the feature axis, eps inside the square root,
    separate (gain, bias) pairs for the attention LN and the FFN LN.
  * act: 0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3))).
  * heads: head h uses columns [h*d_k, (h+1)*d_k) of Q, K, V; scores are scaled by
    1/sqrt(d_k); head outputs are concatenated in head order before W_O.
  * causal: query at position p sees key q iff q <= p (positions within one
    sequence); different sequences of a batch never attend to each other.
  * grouped-query attention ([COST], MQA and GQA): K and V hold g heads of d_k
    columns; query head h reads key/value head h // (n_heads / g) (g is read from
    the widths: K has g d_k columns). g = n_heads is plain multi-head attention.
  * masks of [COST]'s Section 5 (both on top of the causal mask): a window of w
    keys, query p reads keys max(0, p - w + 1) .. p; chunked streaming with chunk
    size C, query p reads every key of its own chunk and of earlier chunks,
    j // C <= p // C.

Every function below is float64 end to end. "Unfused" functions are the plain
definition (full softmax, full [N, d_ff] hidden state); the blockwise function
assembles each row's softmax from per-tile summaries instead, and is used to pin
the former (the pages state that the two give the same values).
"""
from __future__ import annotations

import math

import numpy as np

F64 = np.float64

# The weight names of one layer, in the pages' notation.
WEIGHT_KEYS = ("ln1_g", "ln1_b", "w_q", "w_k", "w_v", "w_o",
               "ln2_g", "ln2_b", "w_1", "w_2")


# ---------------------------------------------------------------------------
# Which keys a query sees
# ---------------------------------------------------------------------------

def visible(q_pos: np.ndarray, k_pos: np.ndarray, causal: bool, window: int = 0,
            chunk: int = 0) -> np.ndarray:
    """[len(q_pos), len(k_pos)] booleans: key position j is visible to query
    position p (positions within one sequence).
      no mask:       every key;
      causal:        j <= p;
      window w > 0:  p - w < j <= p   ([COST] windowed mask: the oldest key query p
                                       reads is max(0, p - w + 1));
      chunk C > 0:   j // C <= p // C ([COST] chunked streaming: every token sees
                                       its whole chunk, earlier chunks stay readable).
    window and chunk apply to the causal setting only and not together."""
    qp = np.asarray(q_pos, np.int64)[:, None]
    kp = np.asarray(k_pos, np.int64)[None, :]
    assert window >= 0 and chunk >= 0 and not (window and chunk)
    if not causal:
        assert window == 0 and chunk == 0
        return np.ones((qp.shape[0], kp.shape[1]), dtype=bool)
    if chunk:
        return kp // chunk <= qp // chunk
    vis = kp <= qp
    if window:
        vis &= kp > qp - window
    return vis


def _group_size(q: np.ndarray, k: np.ndarray, n_heads: int) -> int:
    """Query heads per key/value head: K holds g heads of d_k = q width / n_heads
    columns; g must divide n_heads."""
    dk = q.shape[1] // n_heads
    g = k.shape[1] // dk
    assert g * dk == k.shape[1] and g >= 1 and n_heads % g == 0
    return n_heads // g


def keys_needed(pos_max: int, seq_len: int, causal: bool, chunk: int = 0) -> int:
    """Number of leading keys of a sequence that queries up to position pos_max can see."""
    if not causal:
        return seq_len
    if chunk:
        return min(seq_len, (pos_max // chunk + 1) * chunk)
    return pos_max + 1


# ---------------------------------------------------------------------------
# Row-wise pieces: [BPT] "The structural fact that makes fusion legal"
# ---------------------------------------------------------------------------

def layer_norm(x: np.ndarray, gain: np.ndarray, bias: np.ndarray, eps: float) -> np.ndarray:
    """Normalise each row across the feature axis ([BPT] structural-fact section):
    (x - mean) / sqrt(biased variance + eps) * gain + bias."""
    x = np.asarray(x, dtype=F64)
    mean = x.mean(axis=-1, keepdims=True)
    centred = x - mean
    var = (centred * centred).mean(axis=-1, keepdims=True)
    return centred / np.sqrt(var + eps) * np.asarray(gain, F64) + np.asarray(bias, F64)


def gelu_tanh(u: np.ndarray) -> np.ndarray:
    """The tanh form of GELU used as the FFN's act ([BPT] fused algorithm, h_i line)."""
    u = np.asarray(u, dtype=F64)
    c = math.sqrt(2.0 / math.pi)
    return 0.5 * u * (1.0 + np.tanh(c * (u + 0.044715 * u * u * u)))


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Row softmax with the row maximum subtracted first ([COST] FlashAttention
    paragraph). Entries equal to -inf contribute zero; a row with no finite entry
    is returned as all zeros rather than NaN (the fully-masked-row pitfall in
    [COST]'s pitfalls table; it cannot occur under the causal mask used here)."""
    s = np.asarray(s, dtype=F64)
    m = s.max(axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m)
    tot = e.sum(axis=-1, keepdims=True)
    return np.divide(e, tot, out=np.zeros_like(e), where=tot > 0)


# ---------------------------------------------------------------------------
# Attention: the unfused definition
# ---------------------------------------------------------------------------

def attention_sequence(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_heads: int,
                       causal: bool, q_pos: np.ndarray | None = None,
                       q_chunk: int | None = None, window: int = 0, chunk: int = 0) -> np.ndarray:
    """Multi-head attention of one sequence with a full softmax.

    q: [nq, d] queries at positions q_pos (default 0..nq-1); k, v: [nk, d] keys and
    values at positions 0..nk-1. Returns the concatenated head outputs [nq, d].
    Scores are q k^T / sqrt(d_k) ([BPT] fused algorithm, s line); with causal
    masking key position j is visible to query position p iff j <= p.
    q_chunk, if given, evaluates the query rows in groups of that many rows to
    bound memory; every row's scores, softmax and output are the same (rows are
    independent: [BPT] fused algorithm, outer loop over query blocks).
    window / chunk: the masks of `visible`.
    """
    if q_chunk is not None and q.shape[0] > q_chunk:
        qp = np.arange(q.shape[0]) if q_pos is None else np.asarray(q_pos)
        return np.concatenate([attention_sequence(q[c:c + q_chunk], k, v, n_heads, causal,
                                                  q_pos=qp[c:c + q_chunk], window=window,
                                                  chunk=chunk)
                               for c in range(0, q.shape[0], q_chunk)])
    q = np.asarray(q, F64)
    k = np.asarray(k, F64)
    v = np.asarray(v, F64)
    nq, d = q.shape
    nk = k.shape[0]
    dk = d // n_heads
    if q_pos is None:
        q_pos = np.arange(nq)
    out = np.empty((nq, d), dtype=F64)
    scale = 1.0 / math.sqrt(dk)
    if causal:
        hidden = ~visible(q_pos, np.arange(nk), causal, window, chunk)
    group = _group_size(q, k, n_heads)
    for h in range(n_heads):
        cols = slice(h * dk, (h + 1) * dk)
        kv = slice((h // group) * dk, (h // group + 1) * dk)
        s = (q[:, cols] @ k[:, kv].T) * scale
        if causal:
            s = np.where(hidden, -np.inf, s)
        out[:, cols] = softmax_rows(s) @ v[:, kv]
    return out


def attention_lse_sequence(q: np.ndarray, k: np.ndarray, n_heads: int, causal: bool,
                           q_pos: np.ndarray | None = None, window: int = 0,
                           chunk: int = 0) -> np.ndarray:
    """Per head and query row, the natural log of the softmax normaliser of the
    scaled scores: lse[h, i] = log sum_{j visible to i} exp(q_i . k_j / sqrt(d_k)).

    The forward pass keeps only each row's softmax statistics, a running maximum m
    and the sum l of exp(s - m), so that the backward pass can rebuild the softmax
    without re-deriving the normalisation ([BPT] "The backward pass"; [COST]
    FlashAttention paragraph). Any pair (m, l) of one row determines the same
    m + log l; this is that number, computed from the full row (maximum first).
    q: [nq, d] at positions q_pos (default 0..nq-1); k: [nk, d] at 0..nk-1.
    Returns [n_heads, nq].
    """
    q = np.asarray(q, F64)
    k = np.asarray(k, F64)
    nq, d = q.shape
    nk = k.shape[0]
    dk = d // n_heads
    if q_pos is None:
        q_pos = np.arange(nq)
    scale = 1.0 / math.sqrt(dk)
    out = np.empty((n_heads, nq), dtype=F64)
    if causal:
        hidden = ~visible(q_pos, np.arange(nk), causal, window, chunk)
    group = _group_size(q, k, n_heads)
    for h in range(n_heads):
        cols = slice(h * dk, (h + 1) * dk)
        kv = slice((h // group) * dk, (h // group + 1) * dk)
        s = (q[:, cols] @ k[:, kv].T) * scale
        if causal:
            s = np.where(hidden, -np.inf, s)
        m = s.max(axis=1)
        out[h] = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
    return out


def layer_lse(x: np.ndarray, p: dict, *, seq_len: int, n_heads: int, causal: bool,
              eps: float = 1e-5, window: int = 0, chunk: int = 0) -> np.ndarray:
    """The attention statistics of one layer: [B, n_heads, seq_len], lse of every
    row of every sequence (attention_lse_sequence on Q = LN1(x) W_Q, K = LN1(x) W_K)."""
    x = np.asarray(x, F64)
    p = _as_f64_layer(p)
    rows = x.shape[0]
    assert rows % seq_len == 0
    x1 = layer_norm(x, p["ln1_g"], p["ln1_b"], eps)
    q = x1 @ p["w_q"]
    k = x1 @ p["w_k"]
    return np.stack([attention_lse_sequence(q[s0:s0 + seq_len], k[s0:s0 + seq_len], n_heads, causal,
                                            window=window, chunk=chunk)
                     for s0 in range(0, rows, seq_len)])


def layer_lse_rows(x: np.ndarray, p: dict, rows: np.ndarray, *, seq_len: int, n_heads: int,
                   causal: bool, eps: float = 1e-5, row_chunk: int = 4096, window: int = 0,
                   chunk: int = 0) -> np.ndarray:
    """layer_lse at the given global rows only: [len(rows), n_heads]. Keys are formed
    for the prefix each sampled query can see (in chunks of row_chunk rows, for
    memory), queries for the sampled rows."""
    x = np.asarray(x, F64)
    p = _as_f64_layer(p)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, n_heads), dtype=F64)
    seq_of = rows // seq_len
    for sidx in np.unique(seq_of):
        sel = np.nonzero(seq_of == sidx)[0]
        pos = rows[sel] - sidx * seq_len
        base = sidx * seq_len
        n_keys = keys_needed(int(pos.max()), seq_len, causal, chunk)
        k = np.empty((n_keys, p["w_k"].shape[1]), F64)
        for c0 in range(0, n_keys, row_chunk):
            c1 = min(n_keys, c0 + row_chunk)
            k[c0:c1] = layer_norm(x[base + c0: base + c1], p["ln1_g"], p["ln1_b"], eps) @ p["w_k"]
        q = layer_norm(x[base + pos], p["ln1_g"], p["ln1_b"], eps) @ p["w_q"]
        out[sel] = attention_lse_sequence(q, k, n_heads, causal, q_pos=pos, window=window,
                                          chunk=chunk).T
    return out


def attention_backward_sequence(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
                                n_heads: int, causal: bool, window: int = 0, chunk: int = 0):
    """Gradients of one sequence's attention output A (attention_sequence) with
    respect to Q, K and V, given dA = do. Per head, with S = Q_h K_h^T / sqrt(d_k)
    (masked as in the forward: `visible`) and P = softmax(S) by rows:
        dV_h = P^T dO_h
        dP   = dO_h V_h^T
        dS   = P * (dP - rowsum(P * dP))      (the softmax's Jacobian, row by row)
        dQ_h = dS K_h / sqrt(d_k),   dK_h = dS^T Q_h / sqrt(d_k)
    With g key/value heads (grouped-query attention, g read from the widths), a
    key/value head's dK and dV sum those of the query heads that read it.
    This is the attention part of the backward pass the saved statistics serve
    ([BPT] "The backward pass": each block recomputes s and the attention output
    from the saved (m, l) and accumulates gradients); the plain definition here
    builds the whole P. rowsum(P * dP) equals rowsum(dO * A), the form a block
    recomputation uses. Returns (dq [n, d], dk, dv [n, g d_k]).
    """
    q, k, v, do = (np.asarray(a, F64) for a in (q, k, v, do))
    n, d = q.shape
    dk_ = d // n_heads
    group = _group_size(q, k, n_heads)
    scale = 1.0 / math.sqrt(dk_)
    dq = np.empty_like(q)
    dkk = np.zeros_like(k)
    dv = np.zeros_like(v)
    hidden = ~visible(np.arange(n), np.arange(n), causal, window, chunk) if causal else None
    for h in range(n_heads):
        c = slice(h * dk_, (h + 1) * dk_)
        kv = slice((h // group) * dk_, (h // group + 1) * dk_)
        s = (q[:, c] @ k[:, kv].T) * scale
        if causal:
            s = np.where(hidden, -np.inf, s)
        pm = softmax_rows(s)
        dv[:, kv] += pm.T @ do[:, c]
        dp = do[:, c] @ v[:, kv].T
        ds = pm * (dp - (pm * dp).sum(axis=1, keepdims=True))
        dq[:, c] = ds @ k[:, kv] * scale
        dkk[:, kv] += ds.T @ q[:, c] * scale
    return dq, dkk, dv


def _row_keys(p: int, nk_all: int, causal: bool, window: int, chunk: int) -> np.ndarray:
    """Positions of the keys query p sees (within the first nk_all keys)."""
    keys = np.arange(nk_all)
    return keys[visible(np.array([p]), keys, causal, window, chunk)[0]]


def attention_backward_dq_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
                               n_heads: int, causal: bool, rows: np.ndarray, window: int = 0,
                               chunk: int = 0) -> np.ndarray:
    """dQ of attention_backward_sequence at the given query rows only (a row's dQ
    needs its own row of P and dP, i.e. every key it sees): [len(rows), d]."""
    q, k, v, do = (np.asarray(a, F64) for a in (q, k, v, do))
    rows = np.asarray(rows, dtype=np.int64)
    d = q.shape[1]
    dk_ = d // n_heads
    group = _group_size(q, k, n_heads)
    scale = 1.0 / math.sqrt(dk_)
    out = np.empty((rows.size, d), F64)
    for r_i, r in enumerate(rows):
        keys = _row_keys(int(r), k.shape[0], causal, window, chunk)
        for h in range(n_heads):
            c = slice(h * dk_, (h + 1) * dk_)
            kv = slice((h // group) * dk_, (h // group + 1) * dk_)
            s = (k[keys, kv] @ q[r, c]) * scale
            pm = np.exp(s - s.max())
            pm /= pm.sum()
            dp = v[keys, kv] @ do[r, c]
            ds = pm * (dp - (pm * dp).sum())
            out[r_i, c] = ds @ k[keys, kv] * scale
    return out


def attention_backward_kv_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
                               n_heads: int, causal: bool, rows: np.ndarray, window: int = 0,
                               chunk: int = 0):
    """dK and dV of attention_backward_sequence at the given key rows only:
    (dk, dv), each [len(rows), width of K].

    Key j's gradients sum over the queries p that see it (and, with grouped heads,
    over the query heads of its group): dV_j = sum_p P[p, j] dO_p and dK_j =
    sum_p dS[p, j] Q_p / sqrt(d_k), where P[p, :] is query p's whole softmax row
    (every key it sees) and dS[p, j] = P[p, j] (dO_p . V_j - dO_p . A_p).
    A query whose dO row is zero has dS[p, :] = 0 and P[p, :] dO_p = 0, so it adds
    nothing and is skipped: with dO nonzero on a few rows only, the cost is those
    rows times the sequence length.
    """
    q, k, v, do = (np.asarray(a, F64) for a in (q, k, v, do))
    rows = np.asarray(rows, dtype=np.int64)
    d = q.shape[1]
    dk_ = d // n_heads
    group = _group_size(q, k, n_heads)
    scale = 1.0 / math.sqrt(dk_)
    dk_out = np.zeros((rows.size, k.shape[1]), F64)
    dv_out = np.zeros((rows.size, v.shape[1]), F64)
    live = np.flatnonzero(np.any(do != 0.0, axis=1))
    for p in live:
        keys = _row_keys(int(p), k.shape[0], causal, window, chunk)
        pos_in = {int(j): i for i, j in enumerate(keys)}
        seen = np.array([int(r) in pos_in for r in rows])   # the requested keys query p sees
        if not np.any(seen):
            continue
        idx = np.array([pos_in[int(r)] for r in rows[seen]])
        for h in range(n_heads):
            c = slice(h * dk_, (h + 1) * dk_)
            kv = slice((h // group) * dk_, (h // group + 1) * dk_)
            s = (k[keys, kv] @ q[p, c]) * scale
            pm = np.exp(s - s.max())
            pm /= pm.sum()
            dp = v[keys, kv] @ do[p, c]
            ds = pm * (dp - (pm * dp).sum())
            dv_out[seen, kv] += pm[idx, None] * do[p, c][None, :]
            dk_out[seen, kv] += ds[idx, None] * q[p, c][None, :] * scale
    return dk_out, dv_out

# ---------------------------------------------------------------------------
# The unfused layer (the plain definition the fused loop must reproduce)
# ---------------------------------------------------------------------------

def _as_f64_layer(p: dict) -> dict:
    return {k: np.asarray(p[k], dtype=F64) for k in WEIGHT_KEYS}


def layer_forward(x: np.ndarray, p: dict, *, seq_len: int, n_heads: int, causal: bool,
                  eps: float = 1e-5, return_parts: bool = False, q_chunk: int | None = None,
                  window: int = 0, chunk: int = 0):
    """One pre-LN layer, unfused ([BPT] fused-algorithm section, last paragraph: the
    whole [N, d] attention output first, then a full [N, d_ff] hidden state).

    x: [B*seq_len, d], sequences stacked row-wise. p: weights in (in, out) form.
      x1 = LN1(x);  Q, K, V = x1 W_Q, x1 W_K, x1 W_V
      A  = attention(Q, K, V) per sequence and head
      Y  = x + A W_O
      H  = act(LN2(Y) W_1)          (full [N, d_ff])
      Z  = Y + H W_2
    """
    x = np.asarray(x, F64)
    p = _as_f64_layer(p)
    rows, d = x.shape
    assert rows % seq_len == 0
    x1 = layer_norm(x, p["ln1_g"], p["ln1_b"], eps)
    q = x1 @ p["w_q"]
    k = x1 @ p["w_k"]
    v = x1 @ p["w_v"]
    a = np.empty_like(x)
    for s0 in range(0, rows, seq_len):
        sl = slice(s0, s0 + seq_len)
        a[sl] = attention_sequence(q[sl], k[sl], v[sl], n_heads, causal, q_chunk=q_chunk,
                                   window=window, chunk=chunk)
    y = x + a @ p["w_o"]
    hidden = gelu_tanh(layer_norm(y, p["ln2_g"], p["ln2_b"], eps) @ p["w_1"])
    z = y + hidden @ p["w_2"]
    if return_parts:
        return z, dict(x1=x1, q=q, k=k, v=v, a=a, y=y, hidden=hidden)
    return z


def layer_forward_rows(x: np.ndarray, p: dict, rows: np.ndarray, *, seq_len: int,
                       n_heads: int, causal: bool, eps: float = 1e-5,
                       row_chunk: int = 4096, window: int = 0, chunk: int = 0) -> np.ndarray:
    """The same layer, evaluated only at the given output rows (global row indices).

    Keys and values are computed for every row a sampled query can see (with
    causal masking, the prefix of its sequence up to the last sampled row);
    queries, attention and the row-wise tail only for the sampled rows. Because
    LN, the FFN and the residual adds act on each row alone ([BPT] structural-fact
    section), this equals the corresponding rows of layer_forward.
    K and V are formed in chunks of row_chunk rows purely to bound memory.
    """
    x = np.asarray(x, F64)
    p = _as_f64_layer(p)
    rows = np.asarray(rows, dtype=np.int64)
    total, d = x.shape
    out = np.empty((rows.size, d), dtype=F64)
    seq_of = rows // seq_len
    for sidx in np.unique(seq_of):
        sel = np.nonzero(seq_of == sidx)[0]
        pos = rows[sel] - sidx * seq_len
        base = sidx * seq_len
        n_keys = keys_needed(int(pos.max()), seq_len, causal, chunk)
        k = np.empty((n_keys, p["w_k"].shape[1]), F64)
        v = np.empty((n_keys, p["w_v"].shape[1]), F64)
        for c0 in range(0, n_keys, row_chunk):
            c1 = min(n_keys, c0 + row_chunk)
            xk = layer_norm(x[base + c0: base + c1], p["ln1_g"], p["ln1_b"], eps)
            k[c0:c1] = xk @ p["w_k"]
            v[c0:c1] = xk @ p["w_v"]
        xq = x[base + pos]
        q = layer_norm(xq, p["ln1_g"], p["ln1_b"], eps) @ p["w_q"]
        a = attention_sequence(q, k, v, n_heads, causal, q_pos=pos, window=window, chunk=chunk)
        y = xq + a @ p["w_o"]
        hidden = gelu_tanh(layer_norm(y, p["ln2_g"], p["ln2_b"], eps) @ p["w_1"])
        out[sel] = y + hidden @ p["w_2"]
    return out


def stack_forward(x: np.ndarray, layers: list, *, seq_len: int, n_heads: int,
                  causal: bool, eps: float = 1e-5, window: int = 0, chunk: int = 0) -> np.ndarray:
    """L layers applied in turn, Z_l = layer_l(Z_{l-1}), in float64 with no rounding
    between layers and no final LN."""
    z = np.asarray(x, F64)
    for p in layers:
        z = layer_forward(z, p, seq_len=seq_len, n_heads=n_heads, causal=causal, eps=eps,
                          window=window, chunk=chunk)
    return z


def stack_forward_rows(x: np.ndarray, layers: list, rows: np.ndarray, *, seq_len: int,
                       n_heads: int, causal: bool, eps: float = 1e-5,
                       q_chunk: int | None = None, window: int = 0, chunk: int = 0) -> np.ndarray:
    """Sampled rows of the stack's output: every layer but the last in full (a causal
    row depends on all earlier rows of every earlier layer), the last one at the
    sampled rows only. q_chunk bounds the attention's memory (attention_sequence)."""
    z = np.asarray(x, F64)
    for p in layers[:-1]:
        z = layer_forward(z, p, seq_len=seq_len, n_heads=n_heads, causal=causal, eps=eps,
                          q_chunk=q_chunk, window=window, chunk=chunk)
    return layer_forward_rows(z, layers[-1], rows, seq_len=seq_len, n_heads=n_heads,
                              causal=causal, eps=eps, window=window, chunk=chunk)


# ---------------------------------------------------------------------------
# The layer's backward pass ([BPT] "The backward pass": gradients of the loss with
# respect to the layer input and every parameter, the block's softmax rebuilt
# from its saved statistics; here the plain definition, every intermediate held)
# ---------------------------------------------------------------------------

def layer_norm_backward(x: np.ndarray, gain: np.ndarray, dy: np.ndarray, eps: float):
    """Gradients through y = LN(x) gain + bias given dy = dL/dy, row by row:
    returns (dx, dgain, dbias). With xh = (x - mean) / sqrt(var + eps) and
    g = dy gain: dx = (g - mean(g) - xh mean(g xh)) / sqrt(var + eps);
    dgain = sum over rows of dy xh, dbias = sum over rows of dy."""
    x = np.asarray(x, F64)
    dy = np.asarray(dy, F64)
    mean = x.mean(axis=-1, keepdims=True)
    xc = x - mean
    rstd = 1.0 / np.sqrt((xc * xc).mean(axis=-1, keepdims=True) + eps)
    xh = xc * rstd
    g = dy * np.asarray(gain, F64)
    dx = rstd * (g - g.mean(axis=-1, keepdims=True) - xh * (g * xh).mean(axis=-1, keepdims=True))
    return dx, (dy * xh).sum(axis=0), dy.sum(axis=0)


def gelu_tanh_derivative(u: np.ndarray) -> np.ndarray:
    """d/du of gelu_tanh: 0.5 (1 + tanh z) + 0.5 u (1 - tanh^2 z) dz/du with
    z = c (u + 0.044715 u^3), c = sqrt(2/pi)."""
    u = np.asarray(u, F64)
    c = math.sqrt(2.0 / math.pi)
    t = np.tanh(c * (u + 0.044715 * u ** 3))
    return 0.5 * (1.0 + t) + 0.5 * u * (1.0 - t * t) * c * (1.0 + 3.0 * 0.044715 * u * u)


def layer_backward(x: np.ndarray, p: dict, dz: np.ndarray, *, seq_len: int, n_heads: int,
                   causal: bool, eps: float = 1e-5, window: int = 0, chunk: int = 0) -> dict:
    """Gradients of a loss L through one layer (layer_forward), given dz = dL/dZ.

    Returns a dict with dx (= dL/dX) and, in the pages' (in, out) orientation of
    the weights, dw_q, dw_k, dw_v, dw_o, dw_1, dw_2, and dln1_g, dln1_b, dln2_g,
    dln2_b. Backwards through the forward's steps:
      Z = Y + H W_2:                dY = dZ + (FFN part), dW_2 = H^T dZ, dH = dZ W_2^T
      H = act(U), U = LN2(Y) W_1:   dU = dH act'(U), dW_1 = LN2(Y)^T dU, dLN2 = dU W_1^T
      LN2:                          dY += LN backward of dLN2 (and the LN2 gain / bias)
      Y = X + A W_O:                dX = dY + (attention part), dW_O = A^T dY, dA = dY W_O^T
      attention (per sequence):     dQ, dK, dV = attention_backward_sequence(Q, K, V, dA)
      Q, K, V = LN1(X) W_{Q,K,V}:   dW_Q = LN1(X)^T dQ (and K, V), dLN1 = sum dQ W_Q^T ...
      LN1:                          dX += LN backward of dLN1 (and the LN1 gain / bias)
    window / chunk: the mask of the forward (`visible`); fewer key/value heads than
    query heads come from the widths of W_K and W_V, as in the forward.
    """
    x = np.asarray(x, F64)
    dz = np.asarray(dz, F64)
    p = _as_f64_layer(p)
    rows = x.shape[0]
    assert rows % seq_len == 0 and dz.shape == x.shape
    _z, parts = layer_forward(x, p, seq_len=seq_len, n_heads=n_heads, causal=causal, eps=eps,
                              return_parts=True, window=window, chunk=chunk)
    x1, q, k, v, a, y = (parts[n] for n in ("x1", "q", "k", "v", "a", "y"))
    y2 = layer_norm(y, p["ln2_g"], p["ln2_b"], eps)
    u = y2 @ p["w_1"]
    h = gelu_tanh(u)
    g = {}
    g["dw_2"] = h.T @ dz
    du = (dz @ p["w_2"].T) * gelu_tanh_derivative(u)
    g["dw_1"] = y2.T @ du
    dy_ln, g["dln2_g"], g["dln2_b"] = layer_norm_backward(y, p["ln2_g"], du @ p["w_1"].T, eps)
    dy = dz + dy_ln
    g["dw_o"] = a.T @ dy
    da = dy @ p["w_o"].T
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    for s0 in range(0, rows, seq_len):
        sl = slice(s0, s0 + seq_len)
        dq[sl], dk[sl], dv[sl] = attention_backward_sequence(q[sl], k[sl], v[sl], da[sl], n_heads,
                                                             causal, window, chunk)
    g["dw_q"], g["dw_k"], g["dw_v"] = x1.T @ dq, x1.T @ dk, x1.T @ dv
    dx1 = dq @ p["w_q"].T + dk @ p["w_k"].T + dv @ p["w_v"].T
    dx_ln, g["dln1_g"], g["dln1_b"] = layer_norm_backward(x, p["ln1_g"], dx1, eps)
    g["dx"] = dy + dx_ln
    return g


# ---------------------------------------------------------------------------
# The blockwise form: softmax summaries of key tiles, merged ([BPT] fused
# algorithm; [COST] two-tile running-sum example)
# ---------------------------------------------------------------------------

def softmax_summary(s: np.ndarray, v: np.ndarray):
    """Summary of one set of keys for each score row: (m, l, o) with m the largest
    score, l = sum exp(s - m) and o = sum exp(s - m) v over the keys.

    s: [..., n] scores (-inf for a key the row does not see); v: [n, dv], or
    [..., n, dv] with the leading axes of s (one value matrix per head).
    A row that sees none of the keys gets m = -inf, l = 0, o = 0 (an empty set).
    """
    s = np.asarray(s, F64)
    m = s.max(axis=-1)
    shift = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - shift[..., None])
    return m, e.sum(axis=-1), e @ np.asarray(v, F64)


def merge_summaries(a, b):
    """Summary of the union of two disjoint key sets from their summaries: both
    are rescaled to the larger maximum before adding (the identity behind the
    pages' running sum; an empty set is the neutral element)."""
    (ma, la, oa), (mb, lb, ob) = a, b
    m = np.maximum(ma, mb)
    shift = np.where(np.isfinite(m), m, 0.0)
    wa = np.where(np.isfinite(ma), np.exp(ma - shift), 0.0)
    wb = np.where(np.isfinite(mb), np.exp(mb - shift), 0.0)
    return m, wa * la + wb * lb, wa[..., None] * oa + wb[..., None] * ob


def online_softmax_tiles(s: np.ndarray, v: np.ndarray, tile: int):
    """One score row s [n] with value rows v [n, dv], consumed tile by tile in
    order: the running (m, l, o) is the merge of the summary so far with the next
    tile's ([COST] two-tile example: the rescaled tile sums give the full sum).
    Returns (m, l, o); o / l is the softmax-weighted mean of v."""
    s = np.asarray(s, F64)
    v = np.asarray(v, F64)
    state = (np.float64(-np.inf), np.float64(0.0), np.zeros(v.shape[1], F64))
    for t0 in range(0, s.size, tile):
        state = merge_summaries(state, softmax_summary(s[t0:t0 + tile], v[t0:t0 + tile]))
    m, l, o = state
    return float(m), float(l), o


def _merge_tree(parts: list):
    """Merge summaries pairwise, level by level (any grouping gives the same
    result in exact arithmetic: merging is associative and commutative)."""
    while len(parts) > 1:
        nxt = [merge_summaries(parts[i], parts[i + 1]) for i in range(0, len(parts) - 1, 2)]
        if len(parts) % 2:
            nxt.append(parts[-1])
        parts = nxt
    return parts[0]


def blockwise_layer_forward(x: np.ndarray, p: dict, *, seq_len: int, n_heads: int,
                            causal: bool, block_q: int, block_kv: int,
                            eps: float = 1e-5, window: int = 0, chunk: int = 0) -> np.ndarray:
    """The layer computed the blockwise way, to pin the unfused definition with
    ([BPT] fused algorithm: query blocks are independent, each row's softmax is
    assembled from per-block pieces of the key axis, and the row-wise tail runs on
    the block alone; [BPT] pitfalls: key blocks wholly after the query block are
    never formed).

    Per sequence and query block of block_q rows: the key axis is cut into tiles
    of block_kv keys; only tiles that some row of the block sees are visited; each
    visited tile yields a softmax summary for every (head, row) at once; the
    summaries are merged as a balanced tree (not in key order), and o / l is the
    block's attention output. The block then gets W_O and the residual, LN2, the
    FFN with its [block_q, d_ff] hidden state, and the second residual. Ragged
    tails give shorter last tiles. Slow; for small inputs.
    """
    x = np.asarray(x, F64)
    p = _as_f64_layer(p)
    rows, d = x.shape
    dk = d // n_heads
    z = np.empty_like(x)
    for s0 in range(0, rows, seq_len):
        xs = x[s0:s0 + seq_len]
        x1 = layer_norm(xs, p["ln1_g"], p["ln1_b"], eps)
        kk, vv = x1 @ p["w_k"], x1 @ p["w_v"]
        g = kk.shape[1] // dk
        # [heads, keys, d_k]: query head h reads key/value head h // (n_heads / g)
        kh = np.repeat(kk.reshape(seq_len, g, dk).transpose(1, 0, 2), n_heads // g, axis=0)
        vh = np.repeat(vv.reshape(seq_len, g, dk).transpose(1, 0, 2), n_heads // g, axis=0)
        for i0 in range(0, seq_len, block_q):
            qpos = np.arange(i0, min(seq_len, i0 + block_q))
            qh = (x1[qpos] @ p["w_q"]).reshape(qpos.size, n_heads, dk).transpose(1, 0, 2)
            parts = []
            for j0 in range(0, seq_len, block_kv):
                kpos = np.arange(j0, min(seq_len, j0 + block_kv))
                vis = visible(qpos, kpos, causal, window, chunk)
                if not vis.any():
                    continue                   # no row of the block sees this tile
                s = np.einsum("hqc,hkc->hqk", qh, kh[:, kpos]) / math.sqrt(dk)
                s = np.where(vis[None], s, -np.inf)
                parts.append(softmax_summary(s, vh[:, kpos]))
            _m, l, o = _merge_tree(parts)
            attn = (o / l[..., None]).transpose(1, 0, 2).reshape(qpos.size, d)
            y = xs[qpos] + attn @ p["w_o"]
            hidden = gelu_tanh(layer_norm(y, p["ln2_g"], p["ln2_b"], eps) @ p["w_1"])
            z[s0 + qpos] = y + hidden @ p["w_2"]
    return z


# ---------------------------------------------------------------------------
# Error metrics used by the parity checks
# ---------------------------------------------------------------------------

def max_abs_err(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.max(np.abs(np.asarray(got, F64) - np.asarray(ref, F64)))) if np.size(ref) else 0.0


def rel_fro_err(got: np.ndarray, ref: np.ndarray) -> float:
    ref = np.asarray(ref, F64)
    den = float(np.linalg.norm(ref))
    num = float(np.linalg.norm(np.asarray(got, F64) - ref))
    return num / den if den > 0 else num
