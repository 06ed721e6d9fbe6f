"""CPU oracle for attention over a block-quantized KV cache.

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the CPU-baseline
leg of the benchmark may import this package; the product library never does,
and this package imports nothing from it.

The arithmetic lives in ``kvq_oracle.c`` (plain C, binary32 quantizer and
binary64 attention); this module only compiles it with gcc, loads it with
ctypes and marshals numpy arrays.  Every function cites the page passage it
follows in the C source.

Logical layout (the oracle's own, independent of any GPU layout):
  codes  : uint8 [n_rows][row_bytes]   q8_0: int8 per value; 4-bit codecs: two
           values per byte, even value in the low nibble
  scales : uint16 [n_rows][d // G]     binary16 bit patterns, one per group
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kvq_oracle.c")
LIB = os.path.join(HERE, "libkvq_oracle.so")

# Codec names -> the oracle's own codec numbers (see kvq_oracle.c).
CODECS = {"q8_0": 0, "q4_0": 1, "q4_g64": 2, "f16": 3}
GROUP = {"q8_0": 32, "q4_0": 32, "q4_g64": 64}        # f16: no groups, no scales
QMAX = {"q8_0": 127, "q4_0": 7, "q4_g64": 7}
BITS = {"q8_0": 8, "q4_0": 4, "q4_g64": 4, "f16": 16}

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
               "-std=c11", "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    override = os.environ.get("KVQ_ORACLE_LIBRARY")
    if not override and (not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC)):
        build(force=True)
    lib = ctypes.CDLL(override or LIB)
    P = ctypes.c_void_p
    lib.kvq_oracle_f32_to_f16.argtypes = [ctypes.c_float]
    lib.kvq_oracle_f32_to_f16.restype = ctypes.c_uint16
    lib.kvq_oracle_f32_to_f16_array.argtypes = [P, P, ctypes.c_int64]
    lib.kvq_oracle_f32_to_f16_array.restype = None
    lib.kvq_oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.kvq_oracle_f16_to_f32.restype = ctypes.c_float
    lib.kvq_oracle_row_code_bytes.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.kvq_oracle_row_code_bytes.restype = ctypes.c_int64
    lib.kvq_oracle_quantize_group.argtypes = [ctypes.c_int, P, P, P]
    lib.kvq_oracle_quantize_group.restype = ctypes.c_int
    lib.kvq_oracle_quantize_rows.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, P, P, P]
    lib.kvq_oracle_quantize_rows.restype = ctypes.c_int
    lib.kvq_oracle_dequant_rows.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, P, P, P]
    lib.kvq_oracle_dequant_rows.restype = ctypes.c_int
    lib.kvq_oracle_attend_decode.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int64, ctypes.c_int64, P, P, P,
                                             ctypes.c_double, P, ctypes.c_int, P]
    lib.kvq_oracle_attend_decode.restype = ctypes.c_int
    lib.kvq_oracle_attend_prefill.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int64, ctypes.c_int, ctypes.c_int64,
                                              P, P, P, ctypes.c_double, P, P, ctypes.c_int, P]
    lib.kvq_oracle_attend_prefill.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _check(st: int, what: str) -> None:
    if st != 0:
        raise ValueError(f"oracle {what} failed with status {st}")


# --------------------------------------------------------------------------
# binary16
# --------------------------------------------------------------------------

def f32_to_f16_bits(x: float) -> int:
    return int(_load().kvq_oracle_f32_to_f16(ctypes.c_float(x)))


def f32_to_f16_bits_array(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().kvq_oracle_f32_to_f16_array(_ptr(x), _ptr(out), x.size)
    return out


def f16_bits_to_f32(h: int) -> float:
    return float(_load().kvq_oracle_f16_to_f32(ctypes.c_uint16(h)))


# --------------------------------------------------------------------------
# codec
# --------------------------------------------------------------------------

def row_code_bytes(codec: str, d: int) -> int:
    return d * BITS[codec] // 8


def n_scales(codec: str, d: int) -> int:
    """binary16 scales per row (none for the f16 codec)."""
    return d // GROUP[codec] if codec in GROUP else 0


def quantize_group(codec: str, x) -> tuple[int, np.ndarray]:
    """One group of GROUP[codec] values -> (scale bits, integer codes q_i)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.shape == (GROUP[codec],)
    sb = np.zeros(1, np.uint16)
    q = np.zeros(GROUP[codec], np.int32)
    _check(_load().kvq_oracle_quantize_group(CODECS[codec], _ptr(x), _ptr(sb), _ptr(q)),
           "quantize_group")
    return int(sb[0]), q


def quantize_rows(codec: str, x) -> tuple[np.ndarray, np.ndarray]:
    """fp32 [..., d] rows -> (codes uint8 [..., row_bytes], scales uint16 [..., d/G]; f16: [..., 0])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    d = x.shape[-1]
    lead = x.shape[:-1]
    n = int(np.prod(lead)) if lead else 1
    codes = np.zeros(lead + (row_code_bytes(codec, d),), np.uint8)
    scales = np.zeros(lead + (n_scales(codec, d),), np.uint16)
    _check(_load().kvq_oracle_quantize_rows(CODECS[codec], d, n, _ptr(x), _ptr(codes),
                                            _ptr(scales)), "quantize_rows")
    return codes, scales


def dequant_rows(codec: str, codes, scales, d: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    lead = codes.shape[:-1]
    n = int(np.prod(lead)) if lead else 1
    out = np.zeros(lead + (d,), np.float32)
    _check(_load().kvq_oracle_dequant_rows(CODECS[codec], d, n, _ptr(codes), _ptr(scales),
                                           _ptr(out)), "dequant_rows")
    return out


def quant_dequant(codec: str, x) -> np.ndarray:
    """The values attention sees after quantize-on-append: dequant(quantize(x))."""
    c, s = quantize_rows(codec, x)
    return dequant_rows(codec, c, s, np.asarray(x).shape[-1])


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def attend_decode(q, k_hat, v_hat, length: int, scale: float, heads=None) -> np.ndarray:
    """q [Hq][d]; k_hat/v_hat [Hkv][rows][d] (dequantized); -> [len(heads)][d] fp32."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    k_hat = np.ascontiguousarray(k_hat, dtype=np.float32)
    v_hat = np.ascontiguousarray(v_hat, dtype=np.float32)
    hq, d = q.shape
    hkv, rows, _ = k_hat.shape
    heads = np.arange(hq, dtype=np.int32) if heads is None else np.asarray(heads, np.int32)
    out = np.zeros((len(heads), d), np.float32)
    _check(_load().kvq_oracle_attend_decode(d, hq, hkv, int(length), rows, _ptr(q), _ptr(k_hat),
                                            _ptr(v_hat), float(scale), _ptr(heads), len(heads),
                                            _ptr(out)), "attend_decode")
    return out


def attend_prefill(q, k_hat, v_hat, P: int, scale: float, tokens=None, heads=None) -> np.ndarray:
    """q [T][Hq][d] (bf16 values as fp32); k_hat/v_hat [Hkv][rows][d] holding the prefix
    and the chunk; evaluates the (tokens[i], heads[i]) pairs -> [n][d] fp32.
    With tokens/heads None every (t, h) is evaluated and the result is [T][Hq][d]."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    k_hat = np.ascontiguousarray(k_hat, dtype=np.float32)
    v_hat = np.ascontiguousarray(v_hat, dtype=np.float32)
    T, hq, d = q.shape
    hkv, rows, _ = k_hat.shape
    full = tokens is None
    if full:
        tt, hh = np.meshgrid(np.arange(T), np.arange(hq), indexing="ij")
        tokens, heads = tt.ravel(), hh.ravel()
    tokens = np.ascontiguousarray(tokens, np.int32)
    heads = np.ascontiguousarray(heads, np.int32)
    out = np.zeros((len(tokens), d), np.float32)
    _check(_load().kvq_oracle_attend_prefill(d, hq, hkv, int(P), T, rows, _ptr(q), _ptr(k_hat),
                                             _ptr(v_hat), float(scale), _ptr(tokens),
                                             _ptr(heads), len(tokens), _ptr(out)),
           "attend_prefill")
    return out.reshape(T, hq, d) if full else out
