"""Write tests/golden/stack4_32k_rows.npz: the CPU float64 oracle's output of the
4-layer, 32768-token, d 4096 stack (workload stack4_32k) at its sampled rows.

Only the oracle (oracle/) and the seeded input generator (blockwise_attn_ffn_amd.synth)
are called; nothing comes from the GPU path. The file also stores a SHA-256 of
every input tensor, so the GPU test can check that it regenerated the same inputs.

    python tests/golden/make_stack4_32k.py        # CPU only, ~40 min on 8 cores, ~25 GB RAM
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from blockwise_attn_ffn_amd import synth  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "stack4_32k_rows.npz")


def main() -> None:
    w = synth.WORKLOADS["stack4_32k"]
    t0 = time.time()
    inputs = synth.make_inputs(w, seed=0)
    digest = synth.input_digest(inputs)
    rows = synth.sample_rows(w, w.sample_rows, seed=0)
    x = synth.to_f64(inputs["x"])
    layers = [synth.oracle_weights(layer) for layer in inputs["layers"]]
    del inputs
    print(f"inputs ready ({time.time() - t0:.0f} s), {rows.size} rows", flush=True)
    z = oracle.stack_forward_rows(x, layers, rows, seq_len=w.seq_len, n_heads=w.n_heads,
                                  causal=w.causal, eps=w.ln_eps, q_chunk=1024)
    np.savez_compressed(OUT, rows=rows, z=z, input_sha256=np.array(digest))
    print(f"wrote {OUT} ({time.time() - t0:.0f} s)", flush=True)


if __name__ == "__main__":
    main()
