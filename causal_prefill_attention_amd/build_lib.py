"""Builds libattn_prefill.so for gfx950 with hipcc (no GPU needed).

    python -m causal_prefill_attention_amd.build_lib

The library is written next to this file so that it travels with the
source tree (objects go to ``_build/`` beside it).  Every HIP translation
unit is compiled with packed-fp32 instructions disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libattn_prefill.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["prefill_fwd.hip", "prefill_wide.hip", "prefill_d512.hip", "decode_fwd.hip",
           "decode_scratch.hip", "attn_prefill.cpp"]

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}: {cmd[-1]}")
    noise = [ln for ln in (res.stderr or "").splitlines()
             if ln.strip() and "packed-fp32-ops" not in ln]
    if verbose and noise:
        sys.stderr.write("\n".join(noise) + "\n")


def build(verbose: bool = True) -> str:
    """Compiles every translation unit (in parallel) and links the library."""
    from concurrent.futures import ThreadPoolExecutor

    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                     "-c", os.path.join(CSRC, src), "-o", obj])
    workers = max(1, min(len(cmds), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(workers) as pool:
        for f in [pool.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
