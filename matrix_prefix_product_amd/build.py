"""Compile libmru.so (the MRU scan library) in-tree for gfx950 with hipcc.

Usage:  python -m matrix_prefix_product_amd.build   (or call build()).
Objects go to matrix_prefix_product_amd/_build/, the library to
matrix_prefix_product_amd/libmru.so.  Always recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libmru.so")
SOURCES = ["mru_api.hip", "build_inputs.hip", "build_orth.hip", "scan_valu.hip", "scan_mfma.hip"]

ARCH = "gfx950"
HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-mcode-object-version=5",
    # no packed-fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{os.path.join(ROOT, 'include')}",
    f"-I{CSRC}",
]


def _hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build libmru.so)")
    return path


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every source and link libmru.so; returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [hipcc, *HIP_FLAGS, *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # the host pass does not know the device-only target feature: harmless
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if p.returncode != 0:
            failed.append((src, "\n".join(lines)))
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        msg = "\n\n".join(f"--- {s}\n{t}" for s, t in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout.decode(errors="replace"))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
