"""Builds libsas.so (HIP, gfx950) in-tree, next to this file, and the
stand-alone HBM stream probe that bench.py --stream-floor runs.

    python -m gated_block_sparse_scores_amd.build     # or build() from Python

Every HIP source is compiled with packed-fp32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsas.so")
PROBE = os.path.join(HERE, "stream_probe")  # measurement only, not linked into the library
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

SOURCES = [
    "select.hip",
    "attn_generic.hip",
    "attn_mfma_fwd.hip",
    "attn_mfma_bwd.hip",
    "decode.hip",
    "selector_bwd.hip",
    "sas_api.cpp",
]

ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
    f"-I{INCLUDE}",
]


def _hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build libsas.so)")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    if res.stderr.strip():
        warn = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln]
        if any(w.strip() for w in warn):
            sys.stderr.write(res.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    workers = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking libsas.so failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB)
    cmd = [_hipcc(), *COMMON, "-x", "hip", os.path.join(CSRC, "stream_probe.hip"), "-o",
           PROBE + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"building stream_probe failed:\n{res.stdout}{res.stderr}")
    os.replace(PROBE + ".tmp", PROBE)
    if verbose:
        print(f"built {LIB} and {PROBE}")
    return LIB


if __name__ == "__main__":
    build()
