"""Build libfocus.so (all HIP sources under csrc/) for gfx950, in-tree.

Usage: python attention_delta_token_focus_amd/build.py
(run as a script: the package itself refuses to import until the library
exists)
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIB_DIR, "libfocus.so")

# Packed fp32 VALU ops are switched off for all device code.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; libfocus needs ROCm")
    return exe


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip into lib/libfocus.so; returns its path."""
    os.makedirs(LIB_DIR, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = []
    procs = []
    for src in sources:
        obj = os.path.join(LIB_DIR, os.path.basename(src) + ".o")
        cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-c", src, "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                            stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = False
    for cmd, p in procs:
        out = p.communicate()[0].decode(errors="replace")
        out = "\n".join(l for l in out.splitlines()
                        if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed = True
            sys.stderr.write(" ".join(cmd) + "\n" + out + "\n")
        elif verbose and out.strip():
            sys.stderr.write(out + "\n")
    if failed:
        raise RuntimeError("libfocus: HIP compilation failed")
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs,
           "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    for obj in objs:
        os.remove(obj)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
