"""Build the in-tree C-ABI library ``libbpt.so`` for gfx950 with hipcc.

    python -m blockwise_attn_ffn_amd.build          # compile (always; ~1 min)

The kernels are split over several translation units compiled in parallel,
then linked with the host ABI layer into one shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libbpt.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
# No packed-fp32 instructions: plain fp32 code only.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument", f"-I{INCLUDE}"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", f"-I{INCLUDE}"]

KERNEL_SOURCES = ["k_ln_qkv.hip", "k_gemm.hip", "k_attention.hip", "k_ffn.hip", "k_ffn_coop.hip", "k_pack.hip",
                  "k_attention_bwd.hip", "k_attention_bwd_dkv.hip", "k_ring.hip", "k_noalloc.hip", "k_layer_bwd.hip",
                  "bpt_launch.hip"]
HOST_SOURCES = ["bpt_api.cpp", "bpt_support.cpp", "bpt_host.cpp"]
# Per-source extra flags. The attention backward keeps its matrix-core results in
# ordinary VGPRs (they feed the softmax arithmetic at once); left to itself the
# compiler places them in AGPRs and copies every value back.
EXTRA_FLAGS = {"k_attention_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               # the host (CPU) layer: 8-wide fp32 vectors with fused multiply-add
               "bpt_host.cpp": ["-O3", "-mavx2", "-mfma", "-pthread"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libbpt.so)")


def _run(cmd: list[str]) -> None:
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed ({res.returncode}): {' '.join(cmd)}\n{out}")


def build(verbose: bool = False) -> str:
    """Compile every source and link LIB_PATH. Always rebuilds. Returns the path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    jobs = []
    for src in KERNEL_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        jobs.append([cc, *HIP_FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        jobs.append(["g++", *HOST_FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for f in [ex.submit(_run, j) for j in jobs]:
            f.result()
    objs = [j[-1] for j in jobs]
    tmp = LIB_PATH + ".tmp"
    _run([cc, "-shared", f"--offload-arch={ARCH}", "-pthread", "-o", tmp, *objs])
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
