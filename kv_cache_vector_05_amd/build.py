"""Builds libtq.so (the C-ABI library with the gfx950 HIP kernels) in-tree.

    python -m kv_cache_vector_05_amd.build          # compile and link
    python -m kv_cache_vector_05_amd.build --jobs 8

Each source is compiled by hipcc for gfx950 into _build/ and linked into
kv_cache_vector_05_amd/libtq.so.  Packed-FP32 VALU instructions are disabled
for all device code (``-Xclang -target-feature -Xclang -packed-fp32-ops``);
hipcc's host pass warns that it does not know the feature, which is harmless.
The host table builder is compiled with floating-point contraction off so
that its seeded Gaussians are the plain evaluation of their definition.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libtq.so")
BUILD = os.path.join(ROOT, "_build")

SOURCES = ["tq_host.cpp", "tq_gemm.hip", "tq_encode.hip", "tq_attn.hip", "tq_qprep.hip", "tq_scan.hip", "tq_decode.hip",
           "tq_vq.hip", "tq_noalloc.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; set HIPCC or install ROCm")


def common_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include")]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + common_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd += ["-ffp-contract=off"]
    if src in ("tq_qprep.hip", "tq_scan.hip", "tq_encode.hip", "tq_decode.hip"):
        # keep MFMA accumulators in architectural VGPRs (no AGPR copies in the loop)
        cmd += ["-mllvm", "--amdgpu-mfma-vgpr-form"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stdout}\n{r.stderr}")
    warn = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if verbose and warn:
        print("\n".join(warn), flush=True)
    return obj


def build(jobs: int = 4, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libtq.so failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args(argv)
    print(build(args.jobs, args.verbose))


if __name__ == "__main__":
    sys.exit(main())
