"""A plain device-to-device copy of known size, for calibrating the HBM byte
counters (FETCH_SIZE, WRITE_SIZE) that the kernel profiles report.

    python -m blockwise_attn_ffn_amd.copy_probe [--mib 1024] [--reps 3]

Each repetition copies --mib MiB once (read that many bytes, write that many).
"""
import argparse

import torch


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--mib", type=int, default=1024)
    ap.add_argument("--reps", type=int, default=3)
    a = ap.parse_args()
    n = a.mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(a.reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {a.mib} MiB x {a.reps}", flush=True)


if __name__ == "__main__":
    main()
