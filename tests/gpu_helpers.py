"""Shared helpers of the GPU parity tests (imported by tests, not collected)."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from block_quantized_kv_amd import Layer, kvq_append, layout


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.abs(got - ref).max() / np.abs(ref).max())


def append_rows(layer: Layer, k_rows, v_rows, seq: int, row0: int, chunk: int = 16384):
    """Appends fp32 device rows [n][H][d] at positions row0.. of `seq`."""
    n = k_rows.shape[0]
    dev = k_rows.device
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        pos = torch.arange(row0 + a, row0 + b, dtype=torch.int64, device=dev)
        sq = torch.full((b - a,), seq, dtype=torch.int32, device=dev)
        kvq_append(layer, k_rows[a:b].contiguous(), v_rows[a:b].contiguous(), sq, pos)


def oracle_hat(codec: str, rows_hd: np.ndarray) -> np.ndarray:
    """Oracle quantize-then-dequantize of rows [n][d] -> [n][d]."""
    return oracle.quant_dequant(codec, rows_hd)


def check_plane_bit_exact(plane, seq: int, head: int, rows_nd: np.ndarray, row0: int = 0):
    """GPU plane rows row0.. of (seq, head) equal the oracle's codes and scales."""
    codes, scales = layout.plane_to_rows(plane, seq=seq)
    n = rows_nd.shape[0]
    got_c = codes[0, head, row0:row0 + n]
    got_s = scales[0, head, row0:row0 + n]
    want_c, want_s = oracle.quantize_rows(plane.codec, rows_nd)
    bad = np.nonzero((got_c != want_c).any(1) | (got_s != want_s).any(1))[0]
    assert bad.size == 0, f"{bad.size} rows differ, first at row {row0 + bad[0]}"


# ---- the oracle over many heads at once ------------------------------------
# The oracle is plain single-threaded C; ctypes releases the interpreter lock
# during each call, so independent (kv-head) quantizations and (q-head)
# attentions run side by side on the host's cores.  Nothing about the
# arithmetic changes.

_POOL = None


def pool():
    global _POOL
    if _POOL is None:
        import os
        from concurrent.futures import ThreadPoolExecutor
        oracle._load()  # build/load once, before any thread uses it
        _POOL = ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1)))
    return _POOL


def oracle_decode_all(kc: str, vc: str, q: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray, length: int,
                      scale: float) -> np.ndarray:
    """Every q-head of one query: q fp32 [Hq][d]; k_rows/v_rows fp32 [n][Hkv][d]
    (rows >= length unused) -> binary64 attention over the oracle's own
    quantization of rows [0, length), as fp32 [Hq][d]."""
    Hq, d = q.shape
    Hkv = k_rows.shape[1]
    G = Hq // Hkv

    def hat(g):
        kh = oracle.quant_dequant(kc, np.ascontiguousarray(k_rows[:length, g])[None])
        vh = oracle.quant_dequant(vc, np.ascontiguousarray(v_rows[:length, g])[None])
        return kh, vh

    hats = list(pool().map(hat, range(Hkv)))

    def one(h):
        kh, vh = hats[h // G]
        return oracle.attend_decode(q[h:h + 1], kh, vh, length, scale)[0]

    return np.stack(list(pool().map(one, range(Hq))))


def report(capsys, name: str, err: float, tol: float) -> None:
    """Prints a parity result on the terminal even when output is captured."""
    with capsys.disabled():
        print(f"\n[parity] {name}: max|gpu-oracle|/max|oracle| = {err:.3e} (bar {tol:.0e})", flush=True)
