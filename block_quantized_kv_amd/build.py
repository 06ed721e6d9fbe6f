"""Builds the gfx950 libraries with hipcc, in place:

  libkvq.so        the HIP kernels of the attention path and the C ABI (include/kvq.h)
  libkvq_probe.so  measurement helpers (the GPU's own streaming-read and matrix-core rates) (include/kvq_probe.h), used by the
                   benchmark only; not linked into libkvq.so
  tests/c_abi/decode_step  a plain-C program over the C ABI (the GPU tests run it)

Sources compile in parallel; each library is linked from its own objects."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvq.so")
PROBE_LIB = os.path.join(HERE, "libkvq_probe.so")
SOURCES = ["kvq_api.cpp", "kv_append.hip", "attn_decode.hip", "attn_prefill.hip"]
PROBE_SOURCES = ["probe/stream_probe.hip", "probe/mfma_probe.hip"]
ARCH = "gfx950"
PER_SOURCE_FLAGS: dict = {}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def _common_flags() -> list:
    return ["-O3", "-fPIC", "-std=c++20", f"--offload-arch={ARCH}",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            # no packed fp32 arithmetic anywhere in the device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # LDS and global words are re-read through other types
            "-fno-strict-aliasing",
            "-Wall", "-Wno-unused-function"]


def _compile(src: str, objdir: str, verbose: bool) -> str:
    obj = os.path.join(objdir, src.replace("/", "_").replace(".", "_") + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc()] + _common_flags() + PER_SOURCE_FLAGS.get(src, []) + lang + \
        ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout)
        raise subprocess.CalledProcessError(r.returncode, cmd, r.stdout)
    if verbose and r.stdout:
        print(r.stdout, flush=True)
    return obj


def _link(objs: list, lib: str) -> str:
    tmp = lib + ".tmp"
    subprocess.run([hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs, check=True)
    os.replace(tmp, lib)
    return lib


# A plain-C user of the C ABI (tests/c_abi/decode_step.c): host code only,
# built with the system C compiler against include/kvq.h, libkvq.so and the
# HIP runtime; the GPU tests run it.
C_EXAMPLE_SRC = os.path.join(ROOT, "tests", "c_abi", "decode_step.c")
C_EXAMPLE_BIN = os.path.join(ROOT, "tests", "c_abi", "decode_step")


def build_c_example(verbose: bool = False) -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"), C_EXAMPLE_SRC,
           "-L", HERE, "-lkvq", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../block_quantized_kv_amd", "-Wl,-rpath," + os.path.join(rocm, "lib"),
           "-o", C_EXAMPLE_BIN + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(C_EXAMPLE_BIN + ".tmp", C_EXAMPLE_BIN)
    return C_EXAMPLE_BIN


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source with hipcc and link libkvq.so and libkvq_probe.so,
    then the plain-C example that links libkvq.so."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    jobs = jobs or min(len(srcs), max(1, os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, objdir, verbose), srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    build_c_example(verbose)
    return LIB


# Host sanitizers for the C ABI's host side (argument validation, sizing,
# dispatch): every -fsanitize= reaches the host compiler only (-Xarch_host),
# the device code is built as usual.  The library then expects the clang
# sanitizer runtime to be preloaded (LD_PRELOAD=sanitizer_runtime()).
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]


def sanitizer_runtime() -> str:
    return subprocess.run(["/opt/rocm/llvm/bin/clang", "--print-file-name=libclang_rt.asan-x86_64.so"],
                          capture_output=True, text=True, check=True).stdout.strip()


def build_sanitized(out_dir: str, jobs: int | None = None) -> str:
    """libkvq.so with sanitized host code, in out_dir (not in place)."""
    os.makedirs(out_dir, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, os.cpu_count() or 1))

    def one(src):
        obj = os.path.join(out_dir, src.replace("/", "_").replace(".", "_") + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc()] + _common_flags() + SANITIZE + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            raise subprocess.CalledProcessError(r.returncode, cmd, r.stdout)
        return obj

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(one, SOURCES))
    lib = os.path.join(out_dir, "libkvq.so")
    subprocess.run([hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Xarch_host", "-fsanitize=address",
                    "-Xarch_host", "-fsanitize=undefined", "-o", lib] + objs, check=True)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
