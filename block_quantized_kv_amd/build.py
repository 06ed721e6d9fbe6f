"""Builds libkvq.so (the HIP kernels and the C ABI) for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvq.so")
SOURCES = ["kvq_api.cpp", "kv_append.hip", "attn_decode.hip", "attn_prefill.hip", "stream_probe.hip"]
ARCH = "gfx950"
PER_SOURCE_FLAGS: dict = {}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def build(verbose: bool = False) -> str:
    """Compile every source with hipcc and link libkvq.so in place."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    common = ["-O3", "-fPIC", "-std=c++20", f"--offload-arch={ARCH}",
              "-I", os.path.join(ROOT, "include"), "-I", CSRC,
              # no packed fp32 arithmetic anywhere in the device code
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              # LDS and global words are re-read through other types
              "-fno-strict-aliasing",
              "-Wall", "-Wno-unused-function"]
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".", "_") + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        extra = PER_SOURCE_FLAGS.get(src, [])
        cmd = [hipcc()] + common + extra + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True, stderr=None if verbose else subprocess.PIPE)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
