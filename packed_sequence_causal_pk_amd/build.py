"""Build libpk.so in-tree with hipcc for gfx950 (cross-compiles without a GPU).

    python -m packed_sequence_causal_pk_amd.build
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libpk.so")

SOURCES = ["pk_api.cpp", "pk_meta.hip", "pk_rope.hip", "pk_fwd.hip", "pk_bwd_kv.hip", "pk_bwd_q.hip",
           "pk_aux.hip", "pk_moe.hip", "pk_reload.cpp", "pk_peak.hip", "pk_lora.hip"]
ARCH = "gfx950"

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "--offload-arch=" + ARCH,
    # keep the compiler from emitting packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # a 64-bit value narrowed to 32 bits is an error: __builtin_amdgcn_readfirstlane takes an int,
    # and a pointer passed through it keeps only its low half (a variant of the LoRA tile copy
    # that did so addressed an unmapped page)
    "-Werror=shorten-64-to-32",
]


# Per-source extra flags.  The dK/dV kernel keeps two waves per SIMD busy with long dependent
# product chains; the latency-oriented ("max-ilp") machine scheduler orders its loads and
# products better there (measured: about 2% on the Qwen3-14B-shaped pack), while the forward
# and dQ kernels do better with the default occupancy-oriented one (under max-ilp the dQ kernel
# spills once its tile reads are issued ahead of their products).
SOURCE_FLAGS = {"pk_bwd_kv.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + COMMON_FLAGS + SOURCE_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [hipcc(), "-x", "hip"] + COMMON_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s" % (" ".join(cmd), err))
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every source and link libpk.so next to this file.  Always recompiles."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (" ".join(cmd), res.stderr))
    os.replace(tmp, LIB_PATH)
    if verbose:
        print("built", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build()
