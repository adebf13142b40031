"""Build the HIP library libcattn.so in-tree for gfx950.

    python -m complex_valued_attention_amd.build

Compiles every ``csrc/*.hip`` with hipcc into
``complex_valued_attention_amd/_lib/libcattn.so``.  hipcc cross-compiles, so
this runs on a machine without a GPU.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libcattn.so")
ARCH = os.environ.get("CATTN_OFFLOAD_ARCH", "gfx950")

# Packed fp32 VALU instructions are kept out of every device object.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = []
    with tempfile.TemporaryDirectory(prefix="cattn_build_") as tmp:
        for s in srcs:
            o = os.path.join(tmp, os.path.basename(s) + ".o")
            cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-c", s, "-o", o,
                   "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-command-line-argument",
                   *DEVICE_FLAGS]
            if verbose:
                print(" ".join(cmd), flush=True)
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                sys.stderr.write(r.stdout + r.stderr)
                raise RuntimeError(f"hipcc failed on {os.path.basename(s)}")
            objs.append(o)
        tmp_lib = LIB + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_lib, *objs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("hipcc link failed")
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
