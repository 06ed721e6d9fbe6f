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
