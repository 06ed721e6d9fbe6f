"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the
CPU: the C ABI's host side (argument validation, sizing, dispatch) built with
host sanitizers (block_quantized_kv_amd/build.py, build_sanitized) and the
oracle built likewise (with clang, so that one sanitizer runtime serves both) run the oracle and ABI test
files with the clang sanitizer runtime preloaded; any report fails them.  A
second check plants an out-of-bounds write in an oracle call (an output
buffer one row short) and expects the sanitizer to stop it, so the first
check cannot pass with the sanitizers silently off."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "block_quantized_kv_amd", "_build", "sanitized")


def _newest_source():
    paths = [os.path.join(ROOT, "oracle", "kvq_oracle.c"), os.path.join(ROOT, "include", "kvq.h")]
    for base in (os.path.join(ROOT, "block_quantized_kv_amd", "csrc"),):
        for f in os.listdir(base):
            if f.endswith((".hip", ".cpp", ".h")):
                paths.append(os.path.join(base, f))
    return max(os.path.getmtime(p) for p in paths)


def _build_oracle_sanitized(path):
    src = os.path.join(ROOT, "oracle", "kvq_oracle.c")
    subprocess.run(["/opt/rocm/llvm/bin/clang", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
                    "-std=c11", "-o", path, src, "-lm"], check=True)


@pytest.fixture(scope="module")
def sanitized():
    from block_quantized_kv_amd import build
    lib, olib = os.path.join(OUT, "libkvq.so"), os.path.join(OUT, "libkvq_oracle.so")
    src_t = _newest_source()
    if not os.path.exists(lib) or os.path.getmtime(lib) < src_t:
        build.build_sanitized(OUT)
    if not os.path.exists(olib) or os.path.getmtime(olib) < src_t:
        _build_oracle_sanitized(olib)
    env = dict(os.environ, LD_PRELOAD=build.sanitizer_runtime(), ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", KVQ_LIBRARY=lib, KVQ_ORACLE_LIBRARY=olib)
    return lib, olib, env


def _undefined_symbols(path):
    r = subprocess.run(["nm", "-D", "--undefined-only", path], capture_output=True, text=True, check=True)
    return r.stdout


def test_oracle_and_abi_tests_under_sanitizers(sanitized):
    lib, olib, env = sanitized
    for path in (lib, olib):
        syms = _undefined_symbols(path)
        assert "__asan_" in syms and "__ubsan_handle_" in syms, path  # instrumented
    files = ["tests/test_layout_and_abi.py", "tests/test_oracle_quant.py", "tests/test_oracle_attention.py",
             "tests/test_oracle_fp16.py"]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider"] + files,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    report = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, report
    assert "AddressSanitizer" not in report and "runtime error" not in report, report


def test_sanitizers_stop_a_planted_overflow(sanitized):
    _, _, env = sanitized
    code = """
import ctypes, numpy as np
import oracle
lib = oracle._load()
x = np.ones((4, 64), np.float32)
codes = np.zeros((3, 32), np.uint8)    # one row short: the oracle writes past it
scales = np.zeros((4, 1), np.uint16)
lib.kvq_oracle_quantize_rows(1, 64, 4, x.ctypes.data, codes.ctypes.data, scales.ctypes.data)
print("not stopped")
"""
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0 and "not stopped" not in r.stdout
    assert "heap-buffer-overflow" in r.stderr
