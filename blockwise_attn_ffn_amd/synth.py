"""Seeded synthetic inputs for the BPT layer forward.

This module only draws random numbers and fixes shapes; it holds none of the
layer's arithmetic. The same tensors feed the HIP library and the CPU oracle.

Draw order (one torch CPU generator per call, seeded): X, then for each layer
ln1_g, ln1_b, W_Q, W_K, W_V, W_O, ln2_g, ln2_b, W_1, W_2. LN parameters are drawn
only when a workload randomises them; otherwise gains are 1 and biases 0 and no
numbers are consumed. Every tensor is drawn in float32 with ``torch.randn``,
scaled and shifted, then rounded to the workload's dtype (round to nearest even).

Weights are stored in the library's layout: each projection matrix of the pages'
notation (y = x W, W in (in, out) form) is held transposed, row-major
[out, in], the layout torch.nn.Linear uses. ``oracle_weights`` returns the (in, out)
float64 view the oracle takes.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seq_len: int
    d_model: int
    n_heads: int
    d_ff: int
    causal: bool
    block_q: int
    block_kv: int
    dtype: str            # "f32" or "bf16": X, weights, LN parameters
    n_layers: int = 1
    ln_random: bool = False
    w_std: float = 0.02
    w_std_layer_decay: bool = False   # std 0.02 / sqrt(2 l + 1) for layer l (0-based)
    ln_eps: float = 1e-5
    sample_rows: int = 0  # 0 = compare every row; otherwise sampled rows
    precision: int = 0    # 0: bf16 operands; 1: bf16 (hi, lo) pairs for computed operands
    window: int = 0       # attention window (causal): query p sees keys p - window + 1 .. p
    chunk: int = 0        # chunked streaming (causal): query p sees keys j with j // chunk <= p // chunk
    n_kv_heads: int = 0   # key/value heads (grouped-query attention); 0: n_heads

    @property
    def rows(self) -> int:
        return self.batch * self.seq_len

    @property
    def d_head(self) -> int:
        return self.d_model // self.n_heads

    @property
    def d_kv(self) -> int:
        return (self.n_kv_heads or self.n_heads) * self.d_head

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The workloads the library is measured and checked on.
WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", batch=1, seq_len=256, d_model=128, n_heads=2,
                          d_ff=512, causal=False, block_q=64, block_kv=64, dtype="f32"),
    "gpt2_small": Workload("gpt2_small", batch=8, seq_len=2048, d_model=768, n_heads=12,
                           d_ff=3072, causal=True, block_q=128, block_kv=128, dtype="bf16",
                           ln_random=True),
    "gpt2_medium": Workload("gpt2_medium", batch=64, seq_len=1024, d_model=1024, n_heads=16,
                            d_ff=4096, causal=True, block_q=128, block_kv=128, dtype="bf16"),
    "long_128k": Workload("long_128k", batch=1, seq_len=131072, d_model=2048, n_heads=16,
                          d_ff=8192, causal=True, block_q=128, block_kv=64, dtype="bf16",
                          sample_rows=256),
    "stack4_32k": Workload("stack4_32k", batch=1, seq_len=32768, d_model=4096, n_heads=32,
                           d_ff=16384, causal=True, block_q=128, block_kv=128, dtype="bf16",
                           n_layers=4, w_std_layer_decay=True, sample_rows=128, precision=1),
    # the long-context layer with a 4096-token attention window (the window the
    # transformer-cost page quotes for Mistral 7B)
    "long_128k_w4096": Workload("long_128k_w4096", batch=1, seq_len=131072, d_model=2048,
                                n_heads=16, d_ff=8192, causal=True, block_q=128, block_kv=64,
                                dtype="bf16", sample_rows=256, window=4096),
    # the BPT page's CPU case: a 1B-parameter model's layer (d 2048) on a 4096-token
    # prompt, blocks of 128 rows (the [128, 4d] tile is 2 MB in bf16)
    "slm_1b_4k": Workload("slm_1b_4k", batch=1, seq_len=4096, d_model=2048, n_heads=16,
                          d_ff=8192, causal=True, block_q=128, block_kv=64, dtype="bf16",
                          sample_rows=64),
    # the long-context layer with grouped-query attention: 4 key/value heads
    "long_128k_gqa4": Workload("long_128k_gqa4", batch=1, seq_len=131072, d_model=2048,
                               n_heads=16, d_ff=8192, causal=True, block_q=128, block_kv=64,
                               dtype="bf16", sample_rows=256, n_kv_heads=4),
}

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def _draw(gen: torch.Generator, shape, std: float, mean: float, dtype) -> torch.Tensor:
    t = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t.to(dtype)


def make_inputs(w: Workload, seed: int = 0) -> dict:
    """Draw X [rows, d] and the per-layer weights on the CPU, in the library layout.

    Returns {"x": tensor, "layers": [dict(name -> tensor), ...]} with names
    ln1_g, ln1_b, w_q, w_k, w_v, w_o, ln2_g, ln2_b, w_1, w_2.
    Shapes: LN parameters [d]; w_q/w_o [d, d]; w_k/w_v [d_kv, d] (d_kv = key/value
    heads x d_head, d for multi-head attention); w_1 [d_ff, d]; w_2 [d, d_ff].
    """
    dt = TORCH_DTYPE[w.dtype]
    d, f = w.d_model, w.d_ff
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    x = _draw(gen, (w.rows, d), 1.0, 0.0, dt)
    layers = []
    for li in range(w.n_layers):
        std = w.w_std / math.sqrt(2 * li + 1) if w.w_std_layer_decay else w.w_std

        def ln_pair():
            if w.ln_random:
                return _draw(gen, (d,), 0.05, 1.0, dt), _draw(gen, (d,), 0.02, 0.0, dt)
            return torch.ones(d, dtype=dt), torch.zeros(d, dtype=dt)

        ln1_g, ln1_b = ln_pair()
        wq = _draw(gen, (d, d), std, 0.0, dt)
        wk = _draw(gen, (w.d_kv, d), std, 0.0, dt)
        wv = _draw(gen, (w.d_kv, d), std, 0.0, dt)
        wo = _draw(gen, (d, d), std, 0.0, dt)
        ln2_g, ln2_b = ln_pair()
        w1 = _draw(gen, (f, d), std, 0.0, dt)
        w2 = _draw(gen, (d, f), std, 0.0, dt)
        layers.append(dict(ln1_g=ln1_g, ln1_b=ln1_b, w_q=wq, w_k=wk, w_v=wv, w_o=wo,
                           ln2_g=ln2_g, ln2_b=ln2_b, w_1=w1, w_2=w2))
    return {"x": x, "layers": layers}


LAYER_KEYS = ("ln1_g", "ln1_b", "w_q", "w_k", "w_v", "w_o", "ln2_g", "ln2_b", "w_1", "w_2")


def input_digest(inputs: dict) -> str:
    """SHA-256 over the raw bytes of X and every layer's tensors, in draw order (to
    check that stored expected values belong to exactly these inputs)."""
    h = hashlib.sha256()
    tensors = [inputs["x"]] + [layer[k] for layer in inputs["layers"] for k in LAYER_KEYS]
    for t in tensors:
        h.update(t.detach().contiguous().view(-1).view(torch.uint8).numpy().tobytes())
    return h.hexdigest()


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a CPU tensor's values (bf16 and f32 embed exactly)."""
    return t.detach().to("cpu", torch.float64).numpy()


def oracle_weights(layer: dict) -> dict:
    """float64 weights in the pages' (in, out) orientation, from library-layout tensors."""
    out = {}
    for k, t in layer.items():
        a = to_f64(t)
        out[k] = a.T.copy() if a.ndim == 2 else a
    return out


def sample_rows(w: Workload, count: int, seed: int = 0) -> np.ndarray:
    """Sorted, distinct global row indices to compare at full size: the edges of the
    first blocks and of the sequence, then a uniform draw without replacement."""
    n = w.rows
    fixed = [0, 1, w.block_q - 1, w.block_q, 2 * w.block_q - 1, 2 * w.block_q,
             w.seq_len // 2, w.seq_len - 1, n - 1]
    chosen = sorted({r for r in fixed if 0 <= r < n})
    rng = np.random.default_rng(seed + 1)
    pool = np.setdiff1d(np.arange(n), np.asarray(chosen))
    extra = rng.choice(pool, size=max(0, min(count, n) - len(chosen)), replace=False)
    return np.sort(np.concatenate([np.asarray(chosen, np.int64), extra.astype(np.int64)]))


def make_attention_inputs(batch: int, seq_len: int, d_model: int, seed: int = 0,
                          qk_std: float = 1.0, live_rows: np.ndarray | None = None) -> dict:
    """Draw the attention backward's inputs on the CPU, bf16, each [batch * seq_len,
    d_model] with heads concatenated along the features: Q, K ~ N(0, qk_std^2) (so a
    score q.k / sqrt(d_head) has standard deviation qk_std^2), V, dO ~ N(0, 1), drawn
    in that order from one generator. live_rows, if given, keeps dO only on those
    global rows and zeroes the rest (the gradient is linear in dO; rows without one
    contribute nothing)."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    shape = (batch * seq_len, d_model)
    q = _draw(gen, shape, qk_std, 0.0, torch.bfloat16)
    k = _draw(gen, shape, qk_std, 0.0, torch.bfloat16)
    v = _draw(gen, shape, 1.0, 0.0, torch.bfloat16)
    do = _draw(gen, shape, 1.0, 0.0, torch.bfloat16)
    if live_rows is not None:
        keep = torch.zeros(shape[0], dtype=torch.bool)
        keep[torch.from_numpy(np.asarray(live_rows, np.int64))] = True
        do[~keep] = 0
    return {"q": q, "k": k, "v": v, "do": do}


def make_grad_output(rows: int, d_model: int, seed: int = 0,
                     live_rows: np.ndarray | None = None) -> torch.Tensor:
    """Draw dZ (the gradient of a loss with respect to a layer's output) on the CPU:
    fp32 [rows, d_model], N(0, 1). live_rows, if given, keeps dZ only on those rows
    and zeroes the rest."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed + 7919)
    dz = _draw(gen, (rows, d_model), 1.0, 0.0, torch.float32)
    if live_rows is not None:
        keep = torch.zeros(rows, dtype=torch.bool)
        keep[torch.from_numpy(np.asarray(live_rows, np.int64))] = True
        dz[~keep] = 0
    return dz
