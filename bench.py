#!/usr/bin/env python3
"""Throughput of the fused BPT layer forward on one MI355X.

    python bench.py [--workload long_128k] [--steps K] [--warmup W] [--gpus 1]
    python bench.py --attention-bwd [--workload gpt2_medium] ...

A step is one bpt_layer_fwd (or bpt_stack_fwd) call over one batch of seeded
synthetic input already resident in device memory. W untimed steps, then K
steps timed with device events on the stream the library launches on. Prints
ONE JSON line: algorithmic TFLOP/s (FLOPs from the pages' count: attention
2 d N (N + 1) causal / 4 N^2 d, projections 8 N d^2, FFN 4 N d d_ff), the
fraction of the bf16 dense matrix-core peak, the activation memory, a roofline
entry for the kernel that takes the most time, and the CPU float64 oracle timed
on a bounded sample of the same workload.

Per-kernel durations come from HIP events that the library records on its
launch stream between its kernels during the timed steps themselves. The
roofline's "traffic" (HBM bytes per launch of that kernel) is read from the
counter summaries committed under profiles/ (rocprofv3 FETCH_SIZE and
WRITE_SIZE, calibrated against a plain copy); it is null when no summary
matches the workload or when the kernel's source files have changed since the
counters were taken (a SHA-256 over those files is stored with each entry).

--attention-bwd times bpt_attention_bwd instead, on the workload's attention
shape (batch, seq_len, d_model, n_heads, mask): seeded Gaussian bf16 Q, K, V, dO,
O ~ N(0, 0.1^2), and lse = ln(number of visible keys) (the statistic of uniform
scores); the values do not change the work. FLOPs: 2.5 times the forward
attention's (the score product recomputed, then four gradient products).
"""
from __future__ import annotations

import argparse
import ctypes
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused BPT layer fwd TFLOP/s (1 MI355X) + % bf16 MFMA peak; peak act mem"
PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}   # dense matrix-core peaks of MI355X
# stages of one layer, in launch order, separated by the library's events:
# prep = weight repacking + LN1 into the packed operand; qkv = the projection GEMM
KERNELS = ("prep", "qkv", "attention", "ffn_epilogue")
CSRC = os.path.join(ROOT, "blockwise_attn_ffn_amd", "csrc")
# source files that determine each stage's device code (for the traffic entries)
KERNEL_SOURCES = {
    "prep": ("k_pack.hip", "k_ln_qkv.hip", "ffn_stream.hpp", "bpt_device.hpp"),
    "qkv": ("k_gemm.hip", "bpt_device.hpp"),
    "attention": ("k_attention.hip", "bpt_device.hpp"),
    "ffn_epilogue": ("k_ffn.hip", "k_ffn_coop.hip", "k_gemm.hip", "k_ln_qkv.hip", "ffn_stream.hpp",
                     "bpt_device.hpp", "bpt_internal.h"),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None,
                    help="default: long_128k (the layer forward and --ring), gpt2_medium "
                         "(--attention-bwd, --layer-bwd), slm_1b_4k (--host)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--attention-bwd", action="store_true",
                    help="time the attention backward on the workload's attention shape")
    ap.add_argument("--layer-bwd", action="store_true",
                    help="time the layer backward (bpt_layer_bwd) on the workload's layer shape")
    ap.add_argument("--ring", type=int, default=0,
                    help="time one device's share of Ring Attention over this many devices "
                         "(default workload long_128k: shards of seq_len / devices tokens)")
    ap.add_argument("--host", action="store_true",
                    help="time the host (CPU) fused layer instead (default workload slm_1b_4k)")
    ap.add_argument("--threads", type=int, default=0,
                    help="host layer threads (default: the CPUs available, at most 16)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target duration of the CPU oracle sample")
    return ap.parse_args()


class Hip:
    """hipEvent_t handles through the HIP runtime torch already loaded."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.h.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        assert self.h.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, e):
        self.h.hipEventDestroy(e)


def kernel_flops(w) -> dict:
    """Algorithmic FLOPs per launch of each kernel (matrix products only)."""
    from blockwise_attn_ffn_amd import accounting as A
    b, n, d, f = w.batch, w.seq_len, w.d_model, w.d_ff
    return {"prep": 0,
            "qkv": b * (2 * n * d * d + 4 * n * d * w.d_kv),
            "attention": b * A.attention_flops(n, d, w.causal, w.window, w.chunk),
            "ffn_epilogue": b * (2 * n * d * d + A.ffn_flops(n, d, f))}


def source_digest(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_entry(tag: str, workload: str, kernel: str):
    """A machine-readable entry <!-- tag {...} --> of a committed profile summary for
    this workload and stage, if the stage's source files are unchanged since."""
    digest = source_digest(kernel)
    pat = re.compile(r"<!--\s*" + tag + r"\s*(\{.*?\})\s*-->")
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path) as f:
            for m in pat.finditer(f.read()):
                e = json.loads(m.group(1))
                if (e.get("workload") == workload and e.get("kernel") == kernel
                        and e.get("source_sha256") == digest):
                    return e
    return None


def recorded_traffic(workload: str, kernel: str):
    """HBM bytes per launch (rocprofv3 FETCH_SIZE and WRITE_SIZE, calibrated)."""
    e = recorded_entry("traffic", workload, kernel)
    return int(e["fetch_bytes"]) + int(e["write_bytes"]) if e else None


def recorded_trace_ms(workload: str, kernel: str):
    """Average duration (ms) of the stage's kernels per layer from a committed
    rocprofv3 --kernel-trace --stats summary of the same bench command."""
    e = recorded_entry("trace", workload, kernel)
    return float(e["avg_ms"]) if e else None


def cpu_baseline(w, inputs, target_s: float) -> dict:
    """The oracle, as it stands, on a bounded sample of the workload."""
    import numpy as np
    import oracle
    from blockwise_attn_ffn_amd import accounting as A, synth
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    layers = [synth.oracle_weights(l) for l in inputs["layers"]]
    x = inputs["x"]
    if w.sample_rows == 0 and w.n_layers == 1:
        def run(k):
            xs = synth.to_f64(x[:k * w.seq_len])
            t0 = time.perf_counter()
            oracle.layer_forward(xs, layers[0], seq_len=w.seq_len, n_heads=w.n_heads,
                                 causal=w.causal, eps=w.ln_eps, window=w.window, chunk=w.chunk)
            return time.perf_counter() - t0
        t1 = run(1)
        k = int(max(1, min(w.batch, round(target_s / max(t1, 1e-3)))))
        t = run(k) if k > 1 else t1
        flops = k * A.layer_flops(w.seq_len, w.d_model, w.d_ff, w.causal, w.window, w.chunk, w.d_kv)
        sample = f"{k} of {w.batch} sequences, full layer (unfused, fp64)"
    else:
        # sampled rows of one layer: K, V for the visible prefix, the rest per row
        rows = synth.sample_rows(w, 64 if w.sample_rows else 64, seed=0)
        xs = synth.to_f64(x)
        t0 = time.perf_counter()
        oracle.layer_forward_rows(xs, layers[0], rows, seq_len=w.seq_len, n_heads=w.n_heads,
                                  causal=w.causal, eps=w.ln_eps, window=w.window, chunk=w.chunk)
        t = time.perf_counter() - t0
        d, f = w.d_model, w.d_ff
        nk = int(rows.max()) + 1
        pos = rows % w.seq_len
        if w.chunk:
            seen = np.minimum(w.seq_len, (pos // w.chunk + 1) * w.chunk)
        elif w.window:
            seen = np.minimum(pos + 1, w.window)
        else:
            seen = pos + 1
        flops = 4 * nk * d * w.d_kv + len(rows) * (4 * d * d + 4 * d * f) + int(np.sum(4 * d * seen))
        sample = f"{len(rows)} sampled rows of layer 1 (K/V for {nk} rows), fp64"
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": sample, "seconds": round(t, 3), "flops": int(flops)}


BWD_KERNELS = ("bwd_stats", "bwd_transpose", "bwd_dq", "bwd_dkv")


def cpu_baseline_attention_bwd(w, inp, target_s: float) -> dict:
    """The oracle's attention backward, as it stands, on a bounded sample."""
    import numpy as np
    import oracle
    from blockwise_attn_ffn_amd import accounting as A, synth
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    n, d, h = w.seq_len, w.d_model, w.n_heads
    if n <= 4096:
        def run(k):
            t0 = time.perf_counter()
            for s_ in range(k):
                r = slice(s_ * n, (s_ + 1) * n)
                oracle.attention_backward_sequence(*(synth.to_f64(inp[x][r]) for x in ("q", "k", "v", "do")),
                                                   h, w.causal)
            return time.perf_counter() - t0
        t1 = run(1)
        k = int(max(1, min(w.batch, round(target_s / max(t1, 1e-3)))))
        t = run(k) if k > 1 else t1
        flops = k * A.attention_bwd_flops(n, d, w.causal)
        sample = f"{k} of {w.batch} sequences, every head (full softmax, fp64)"
    else:
        rows = np.sort(np.random.default_rng(0).choice(n, 16, replace=False))
        q, k_, v, g = (synth.to_f64(inp[x][:n]) for x in ("q", "k", "v", "do"))
        t0 = time.perf_counter()
        oracle.attention_backward_dq_rows(q, k_, v, g, h, w.causal, rows)
        t = time.perf_counter() - t0
        # per row and visible key: scores, dP and the dQ product (3 x 2 d FLOPs)
        flops = int(sum(6 * d * ((r + 1) if w.causal else n) for r in rows))
        sample = f"dQ of {len(rows)} sampled rows of sequence 0 (fp64)"
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": sample, "seconds": round(t, 3), "flops": int(flops)}


def bench_attention_bwd(args, w):
    import torch
    from blockwise_attn_ffn_amd import accounting as A, bpt, synth

    b, n, d, h = w.batch, w.seq_len, w.d_model, w.n_heads
    inp = synth.make_attention_inputs(b, n, d, seed=args.seed)
    dev = {k: t.cuda() for k, t in inp.items()}
    gen = torch.Generator(device="cpu")
    gen.manual_seed(args.seed + 1)
    o = (torch.randn(b * n, d, generator=gen) * 0.1).to(torch.bfloat16).cuda()
    cnt = torch.arange(1, n + 1, dtype=torch.float64) if w.causal else torch.full((n,), float(n),
                                                                                  dtype=torch.float64)
    lse = cnt.log().float().expand(b, h, n).contiguous().cuda()
    desc = bpt.make_attn_desc(batch=b, seq_len=n, d_model=d, n_heads=h, causal=w.causal)
    ws_bytes = bpt.attention_bwd_workspace_bytes(desc)
    ws = bpt.alloc_workspace(ws_bytes)
    outs = [torch.empty(b * n, d, dtype=torch.float32, device="cuda") for _ in range(3)]
    stream = torch.cuda.current_stream()
    hip = Hip()
    evs = [[hip.event() for _ in range(5)] for _ in range(args.steps)]

    def step(events=None):
        if events is None:
            bpt.attention_bwd(desc, dev["q"], dev["k"], dev["v"], o, dev["do"], lse, *outs, ws, stream)
        else:
            bpt.attention_bwd_profiled(desc, dev["q"], dev["k"], dev["v"], o, dev["do"], lse, *outs, ws,
                                       events, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        step(evs[i])
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    per_kernel = {k: 0.0 for k in BWD_KERNELS}
    for ev in evs:
        for i, k in enumerate(BWD_KERNELS):
            per_kernel[k] += hip.elapsed_ms(ev[i], ev[i + 1]) / args.steps
        for e in ev:
            hip.destroy(e)
    flops = b * A.attention_bwd_flops(n, d, w.causal)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS["bf16"]
    # products each kernel runs over the visible (query, key) pairs, each half of
    # the forward attention's two: dQ kernel S, dP, dQ; dK / dV kernel S, dP, dV, dK
    half = b * A.attention_flops(n, d, w.causal) // 2
    kf = {"bwd_stats": 0, "bwd_transpose": 0, "bwd_dq": 3 * half, "bwd_dkv": 4 * half}
    dom = max(BWD_KERNELS, key=lambda k: per_kernel[k])
    achieved = kf[dom] / (per_kernel[dom] * 1e-3) / 1e12
    line = {
        "metric": "attention backward TFLOP/s (1 MI355X) + % bf16 MFMA peak",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded Gaussian Q, K, V, dO, O)",
        "config": {"workload": w.name + " attention backward", "batch": b, "seq_len": n,
                   "d_model": d, "n_heads": h, "causal": w.causal, "parallelism": "none"},
        "pct_peak": round(100 * tflops / peak, 2), "flops_per_step": flops,
        "kernel_ms": {k: round(v, 4) for k, v in per_kernel.items()},
        "kernel_tflops": {k: round(kf[k] / (per_kernel[k] * 1e-3) / 1e12, 2)
                          for k in BWD_KERNELS if kf[k] and per_kernel[k] > 0},
        "memory": {"workspace_bytes": ws_bytes},
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None,
                     "avg_ms": round(per_kernel[dom], 4), "flops_per_launch": kf[dom]},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_attention_bwd(w, inp, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def bench_layer_bwd(args, w):
    """The layer backward: one forward with lse (untimed), W warm-up backward calls,
    then K timed calls, each writing dX and every parameter gradient."""
    import torch
    from blockwise_attn_ffn_amd import accounting as A, bpt, synth

    assert w.n_layers == 1
    inputs = synth.make_inputs(w, seed=args.seed)
    dev = {"x": inputs["x"].cuda(), "layer": {k: t.cuda() for k, t in inputs["layers"][0].items()}}
    desc = bpt.desc_for(w, out_dtype="f32")
    z = torch.empty((w.rows, w.d_model), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.batch, w.n_heads, w.seq_len), dtype=torch.float32, device="cuda")
    ws = bpt.alloc_workspace(bpt.layer_workspace_bytes(desc))
    bpt.layer_fwd_lse(desc, dev["x"], dev["layer"], z, lse, ws)
    torch.cuda.synchronize()
    del ws
    dz = synth.make_grad_output(w.rows, w.d_model, seed=args.seed).cuda()
    dx = torch.empty_like(dz)
    grads = {k: torch.empty(t.shape, dtype=torch.float32, device="cuda") for k, t in dev["layer"].items()}
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    ws_bytes = bpt.layer_bwd_workspace_bytes(desc)
    bws = bpt.alloc_workspace(ws_bytes)
    stream = torch.cuda.current_stream()

    def step():
        bpt.layer_bwd(desc, dev["x"], dev["layer"], lse, dz, dx, grads, bws, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    peak_extra = torch.cuda.max_memory_allocated() - base
    n, d, f = w.seq_len, w.d_model, w.d_ff
    flops = w.batch * A.layer_bwd_flops(n, d, f, w.causal)
    executed = flops + w.batch * A.layer_flops(n, d, f, w.causal)
    tflops = flops / (ms * 1e-3) / 1e12
    block_rows = min(w.rows, max(128, ((1 << 26) // f) // 128 * 128))
    line = {
        "metric": "layer backward TFLOP/s (1 MI355X) + % bf16 MFMA peak",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded Gaussian X, weights, dZ)",
        "config": {"workload": w.name + " layer backward", "batch": w.batch, "seq_len": n,
                   "d_model": d, "n_heads": w.n_heads, "d_ff": f, "causal": w.causal,
                   "parallelism": "none"},
        "pct_peak": round(100 * tflops / PEAK_TFLOPS["bf16"], 2), "flops_per_step": flops,
        "executed_tflops": round(executed / (ms * 1e-3) / 1e12, 2),
        "flops_note": "value counts the backward's products (2x the forward's dense products, "
                      "2.5x its attention products); executed_tflops adds the forward recomputed "
                      "from X and lse",
        "memory": {"workspace_bytes": ws_bytes, "peak_allocated_during_backward": int(peak_extra),
                   "ffn_block_rows": block_rows,
                   "largest_d_ff_wide_buffer_bytes": block_rows * f * 4,
                   "rows_x_d_ff_bf16_bytes": w.rows * f * 2},
    }
    print(json.dumps(line), flush=True)


def bench_host(args, w):
    """The host (CPU) fused layer: W warm-up calls, then K timed calls (wall clock)."""
    import torch
    from blockwise_attn_ffn_amd import accounting as A, bpt, synth

    n_threads = args.threads or max(1, min(16, len(os.sched_getaffinity(0))))
    inputs = synth.make_inputs(w, seed=args.seed)
    desc = bpt.desc_for(w, out_dtype="f32")
    ws_bytes = bpt.layer_host_workspace_bytes(desc, n_threads)
    ws = torch.empty(ws_bytes, dtype=torch.uint8)
    z = torch.empty((w.rows, w.d_model), dtype=torch.float32)
    for _ in range(args.warmup):
        bpt.layer_fwd_host(desc, inputs["x"], inputs["layers"][0], z, ws, n_threads)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        bpt.layer_fwd_host(desc, inputs["x"], inputs["layers"][0], z, ws, n_threads)
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    flops = A.workload_flops(w.batch, w.seq_len, w.d_model, w.d_ff, w.causal, 1, w.window, w.chunk,
                             w.d_kv)
    line = {
        "metric": "fused BPT layer fwd on the host CPU, TFLOP/s (fp32 arithmetic)",
        "value": round(flops / (ms * 1e-3) / 1e12, 4), "unit": "TFLOP/s", "n_gpus": 0,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded Gaussian X and weights, random-init)",
        "config": {"workload": w.name + " (host)", "batch": w.batch, "seq_len": w.seq_len,
                   "d_model": w.d_model, "n_heads": w.n_heads, "d_ff": w.d_ff, "causal": w.causal,
                   "block_q": w.block_q, "input_dtype": w.dtype, "threads": n_threads},
        "flops_per_step": flops,
        "memory": {"workspace_bytes": ws_bytes,
                   "ffn_hidden_unfused_bytes": w.rows * w.d_ff * 2,
                   "ffn_hidden_tile_bytes_per_thread": w.block_q * 512 * 4},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, inputs, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def bench_ring(args, w, R):
    """The last device of an R-device ring (it meets every shard: R - 1 earlier ones
    unmasked and its own causal): R steps + R merges per timed iteration; also one
    unmasked step alone."""
    import torch
    from blockwise_attn_ffn_amd import accounting as A, bpt, synth

    n = w.seq_len // R
    d, h = w.d_model, w.n_heads
    gen = torch.Generator(device="cpu")
    gen.manual_seed(args.seed)
    shards = {x: [(torch.randn(n, d, generator=gen)).to(torch.bfloat16).cuda() for _ in range(R)]
              for x in ("q", "k", "v")}
    desc_full = bpt.make_attn_desc(batch=1, seq_len=n, d_model=d, n_heads=h, causal=False)
    desc_diag = bpt.make_attn_desc(batch=1, seq_len=n, d_model=d, n_heads=h, causal=True)
    ws = bpt.alloc_workspace(bpt.attention_fwd_workspace_bytes(desc_full))
    o = torch.empty(n, d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(1, h, n, dtype=torch.float32, device="cuda")
    o_acc = torch.zeros(n, d, dtype=torch.float32, device="cuda")
    lse_acc = torch.empty(1, h, n, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    q = shards["q"][R - 1]

    def ring_steps():
        lse_acc.fill_(float("-inf"))
        for s_ in range(R):
            dsc = desc_diag if s_ == R - 1 else desc_full
            bpt.attention_fwd(dsc, q, shards["k"][s_], shards["v"][s_], o, lse, ws, stream)
            bpt.attention_merge(desc_full, o_acc, lse_acc, o, lse, stream)

    # the shards as they travel: packed once by their owners (outside the timed share)
    kv = []
    for s_ in range(R):
        buf = bpt.alloc_workspace(bpt.ring_kv_bytes(desc_diag))
        bpt.ring_pack_kv(desc_diag, shards["k"][s_], shards["v"][s_], buf, stream)
        kv.append(buf)
    ws_share = bpt.alloc_workspace(bpt.ring_share_workspace_bytes(desc_diag))

    def ring():
        bpt.ring_share_fwd(desc_diag, R - 1, q, kv, o, lse, ws_share, stream)

    def one_step():
        bpt.attention_fwd(desc_full, q, shards["k"][0], shards["v"][0], o, lse, ws, stream)

    def timed(fn, steps):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(steps):
            fn()
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    ms_ring = timed(ring, args.steps)
    ms_ring_steps = timed(ring_steps, args.steps)
    ms_step = timed(one_step, args.steps)
    flops_ring = (R - 1) * A.attention_flops(n, d, False) + A.attention_flops(n, d, True)
    flops_step = A.attention_flops(n, d, False)
    line = {
        "metric": "Ring Attention, one device's share: TFLOP/s of its steps (1 MI355X)",
        "value": round(flops_ring / (ms_ring * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_ring, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded Gaussian Q, K, V)",
        "config": {"workload": f"{w.name} over {R} devices, the last device", "shard_tokens": n,
                   "d_model": d, "n_heads": h, "ring_steps": R, "parallelism": "none (one device's share)"},
        "flops_per_step": flops_ring,
        "share_path": "bpt_ring_share_fwd: Q packed once, shards arrive packed, steps merged in the "
                      "attention kernel",
        "step_and_merge_path_ms": round(ms_ring_steps, 3),
        "one_unmasked_step": {"ms": round(ms_step, 3), "flops": flops_step,
                              "tflops": round(flops_step / (ms_step * 1e-3) / 1e12, 2)},
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.ring:
        import torch
        from blockwise_attn_ffn_amd import synth
        if not torch.cuda.is_available():
            print(json.dumps({"error": "no GPU visible"}))
            sys.exit(1)
        wl = args.workload or "long_128k"
        return bench_ring(args, synth.WORKLOADS[wl], args.ring)
    if args.host:
        from blockwise_attn_ffn_amd import synth
        wl = args.workload or "slm_1b_4k"
        return bench_host(args, synth.WORKLOADS[wl])
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.attention_bwd:
        import torch
        from blockwise_attn_ffn_amd import synth
        if not torch.cuda.is_available():
            print(json.dumps({"error": "no GPU visible"}))
            sys.exit(1)
        return bench_attention_bwd(args, synth.WORKLOADS[args.workload or "gpt2_medium"])
    if args.layer_bwd:
        import torch
        from blockwise_attn_ffn_amd import synth
        if not torch.cuda.is_available():
            print(json.dumps({"error": "no GPU visible"}))
            sys.exit(1)
        return bench_layer_bwd(args, synth.WORKLOADS[args.workload or "gpt2_medium"])

    import torch
    from blockwise_attn_ffn_amd import accounting as A, bpt, synth

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    w = synth.WORKLOADS[args.workload or "long_128k"]
    torch.cuda.init()
    free_start, total_mem = torch.cuda.mem_get_info()

    inputs = synth.make_inputs(w, seed=args.seed)
    dev_x = inputs["x"].cuda()
    dev_layers = [{k: v.cuda() for k, v in l.items()} for l in inputs["layers"]]
    out_dtype = "f32"
    desc = bpt.desc_for(w, out_dtype=out_dtype)
    ws_bytes = (bpt.layer_workspace_bytes(desc) if w.n_layers == 1
                else bpt.stack_workspace_bytes(desc, w.n_layers))
    ws = bpt.alloc_workspace(ws_bytes)
    z = torch.empty((w.rows, w.d_model), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    hip = Hip()
    single = w.n_layers == 1
    # one set of 5 events per timed step: the library records them on its launch
    # stream between its kernels, so per-kernel durations come from the timed steps
    evs = [[hip.event() for _ in range(5)] for _ in range(args.steps if single else 0)]

    def step(events=None):
        if single:
            if events is not None:
                bpt.layer_fwd_profiled(desc, dev_x, dev_layers[0], z, ws, events, stream)
            else:
                bpt.layer_fwd(desc, dev_x, dev_layers[0], z, ws, stream)
        else:
            bpt.stack_fwd(desc, dev_x, dev_layers, z, ws, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K whole steps
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(evs[i] if single else None)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    free_after, _ = torch.cuda.mem_get_info()

    per_kernel = {k: 0.0 for k in KERNELS}
    for ev in evs:
        for i, k in enumerate(KERNELS):
            per_kernel[k] += hip.elapsed_ms(ev[i], ev[i + 1]) / args.steps
        for e in ev:
            hip.destroy(e)

    breakdown_note = None
    if not single:
        # Per-stage breakdown of a stack: after the timed steps, one profiled layer
        # call per layer (its weights, the bf16 X, the stack's workspace) runs the
        # same kernels on the same shapes; the stages are summed over the layers.
        # Untimed as a whole; the stack's ms_per_step above is the timed figure.
        n_prof = 2
        pevs = [[[hip.event() for _ in range(5)] for _ in range(w.n_layers)] for _ in range(n_prof + 1)]
        for rep_ in range(n_prof + 1):
            for li in range(w.n_layers):
                bpt.layer_fwd_profiled(desc, dev_x, dev_layers[li], z, ws, pevs[rep_][li], stream)
        torch.cuda.synchronize()
        for rep_ in range(1, n_prof + 1):          # the first pass is a warm-up
            for li in range(w.n_layers):
                for i, k in enumerate(KERNELS):
                    per_kernel[k] += hip.elapsed_ms(pevs[rep_][li][i], pevs[rep_][li][i + 1]) / n_prof
        for rep_ in pevs:
            for lv in rep_:
                for e in lv:
                    hip.destroy(e)
        breakdown_note = (f"stages from {n_prof} profiled passes of {w.n_layers} single-layer calls "
                          "(same kernels and shapes as the stack), summed over the layers")

    total_flops = A.workload_flops(w.batch, w.seq_len, w.d_model, w.d_ff, w.causal, w.n_layers,
                                   w.window, w.chunk, w.d_kv)
    tflops = total_flops / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    kf = {k: v * w.n_layers for k, v in kernel_flops(w).items()}   # per step (all layers)
    roofline = None
    if any(v > 0 for v in per_kernel.values()):
        dom = max(KERNELS, key=lambda k: per_kernel[k])
        achieved = kf[dom] / (per_kernel[dom] * 1e-3) / 1e12
        roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                    "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                    "traffic": recorded_traffic(w.name, dom), "traffic_unit": "bytes",
                    "avg_ms": round(per_kernel[dom], 4), "flops_per_launch": kf[dom],
                    "launches_per_step": w.n_layers}
        # the same stage's average duration in the committed kernel-trace summary
        tr = recorded_trace_ms(w.name, dom)
        if tr:
            roofline.update({"trace_avg_ms": round(tr, 4),
                             "trace_frac": round(kf[dom] / (tr * 1e-3) / 1e12 / peak, 4),
                             "event_over_trace": round(per_kernel[dom] / tr, 4)})
    act_bytes = ws_bytes + dev_x.numel() * dev_x.element_size() + z.numel() * z.element_size()
    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded Gaussian X and weights, random-init)",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": w.seq_len,
                   "d_model": w.d_model, "n_heads": w.n_heads, "d_ff": w.d_ff,
                   "causal": w.causal, "block_q": w.block_q, "block_kv": w.block_kv,
                   "n_layers": w.n_layers, "out_dtype": out_dtype, "parallelism": "none",
                   "precision": ("bf16 pairs (hi + lo) for computed operands" if w.precision
                                 else "bf16 operands")},
        "pct_peak": round(100 * tflops / peak, 2),
        "flops_per_step": total_flops,
        "kernel_ms": {k: round(v, 4) for k, v in per_kernel.items()},
        "kernel_tflops": {k: round(kf[k] / (per_kernel[k] * 1e-3) / 1e12, 2)
                          for k in KERNELS if per_kernel[k] > 0 and kf[k] > 0},
        "memory": {"workspace_bytes": ws_bytes, "activation_bytes": act_bytes,
                   "device_bytes_used": int(free_start - free_after),
                   "ffn_hidden_unfused_bytes": w.rows * w.d_ff * 2,
                   "logits_one_head_bytes": w.batch * w.seq_len * w.seq_len * 2},
        "roofline": roofline,
    }
    if breakdown_note:
        line["kernel_ms_note"] = breakdown_note
    if w.precision:
        line["precision_note"] = ("bf16 pairs: each activation operand is hi + lo bf16, so the "
                                  "projections and FFN run two matrix products and attention three "
                                  "per algorithmic product; plain bf16 misses max|err| 2e-2 at this "
                                  "width (the pages' tolerance), which is why the pairs are used")
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, inputs, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
