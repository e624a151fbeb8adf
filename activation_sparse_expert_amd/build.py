"""Compile the HIP library (libmoe_sel.so) in-tree for gfx950 with hipcc.

Usage: ``python -m activation_sparse_expert_amd.build`` (or ``build()``).
Always recompiles. Objects go to ``_build/``; the library lands next to this
file so that it travels with the source tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe_sel.so")
ARCH = "gfx950"

COMMON = ["-std=c++17", "-O3", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-result"]
# Device code: no packed-fp32 instructions; keep fp32 denormals (IEEE); the
# pinned score code turns contraction off locally with a pragma.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-flush-denormals-to-zero", "-munsafe-fp-atomics"]
# Host preparation: exact statistics must not be contracted or reassociated.
HOST_EXACT = ["-ffp-contract=off", "-fno-fast-math", "-march=x86-64-v3"]

SOURCES = [
    ("kernels.hip", DEVICE),
    ("fused.hip", DEVICE),
    ("lowrank_device.hip", DEVICE),
    ("sketch_device.hip", DEVICE),
    ("decode_glue.hip", DEVICE),
    ("debug_device.hip", DEVICE),
    ("api.cpp", DEVICE),
    ("prepare_host.cpp", HOST_EXACT),
    ("fault.cpp", HOST_EXACT),
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build the HIP library)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(ln for ln in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src, flags in SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") or flags is DEVICE else []
        _run([hipcc, *COMMON, *flags, *lang, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, "-pthread"], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
