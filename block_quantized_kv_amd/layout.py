"""Host-side description of the in-block permutation of the cache planes
(the same permutation the HIP kernels use; see csrc/kvq_layout.h).

Used to read GPU planes back in plain row-major order: codes of row r as
``row_bytes`` bytes (q8_0: one int8 per channel; 4-bit: two channels per byte,
even channel in the low nibble) and ``head_dim / G`` binary16 scales."""
from __future__ import annotations

import numpy as np

BLOCK_ROWS = 32
GROUP = {"q8_0": 32, "q4_0": 32, "q4_g64": 64}   # f16: no scales


def _is8(codec):
    return codec == "q8_0"


def row_bytes(codec, d):
    return 2 * d if codec == "f16" else d if _is8(codec) else d // 2


def n_scales(codec, d):
    return 0 if codec == "f16" else d // GROUP[codec]


def _lane_byte_offset(LB, lane, b):
    W = min(LB, 16)
    return (b // W) * (64 * W) + lane * W + (b % W)


def _slot_nibble(s):
    return (s >> 1) + 4 * (s & 1)


def code_positions(codec: str, role: str, d: int):
    """(byte, shift) arrays of shape [32][d]: where the code of block row j,
    channel c lives inside a block."""
    byte, shift = _code_positions(codec, role, d)
    shape = (BLOCK_ROWS, d)
    return np.broadcast_to(byte, shape).copy(), np.broadcast_to(shift, shape).copy()


def _code_positions(codec: str, role: str, d: int):
    j = np.arange(BLOCK_ROWS)[:, None]
    c = np.arange(d)[None, :]
    if role == "k":
        tau, i = j >> 4, j & 15
        t, kq, s = c >> 5, (c & 31) >> 3, c & 7
        lane = i + 16 * kq
        tile = tau * 16 * row_bytes(codec, d)
        if codec == "f16":   # byte position of the value's low byte
            return tile + _lane_byte_offset(d // 2, lane, 16 * t + 2 * s), np.zeros_like(lane + tile)
        if _is8(codec):
            LB = d // 4
            return tile + _lane_byte_offset(LB, lane, 8 * t + s), np.zeros_like(lane + tile)
        LB = d // 8
        p = _slot_nibble(s)
        return tile + _lane_byte_offset(LB, lane, 4 * t + (p >> 1)), 4 * (p & 1) + 0 * tile
    cb, c16 = c >> 4, c & 15
    kq, s = (j & 15) >> 2, 4 * (j >> 4) + (j & 3)
    lane = c16 + 16 * kq
    if codec == "f16":
        return _lane_byte_offset(d, lane, 16 * cb + 2 * s), np.zeros_like(lane)
    if _is8(codec):
        LB = d // 2
        return _lane_byte_offset(LB, lane, 8 * cb + s), np.zeros_like(lane)
    LB = d // 4
    p = _slot_nibble(s)
    return _lane_byte_offset(LB, lane, 4 * cb + (p >> 1)), 4 * (p & 1)


def scale_positions(codec: str, role: str, d: int):
    """Index (binary16 units) of the scale of block row j, group g: [32][ng]."""
    ng = n_scales(codec, d)
    j = np.arange(BLOCK_ROWS)[:, None]
    g = np.arange(ng)[None, :]
    if role == "k":
        tau, i = j >> 4, j & 15
        return tau * 16 * ng + (i >> 2) * 4 * ng + g * 4 + (i & 3)
    kq, s = (j & 15) >> 2, 4 * (j >> 4) + (j & 3)
    return kq * 8 * ng + g * 8 + s


def unpack_codes(codec: str, role: str, d: int, blocks: np.ndarray) -> np.ndarray:
    """blocks uint8 [..., n_blocks, 32 * row_bytes] -> row-major codes
    uint8 [..., n_blocks * 32, row_bytes]."""
    blocks = np.asarray(blocks, np.uint8)
    lead = blocks.shape[:-2]
    nb = blocks.shape[-2]
    byte, shift = code_positions(codec, role, d)
    if codec == "f16":
        # each value's two bytes (little-endian) in channel order
        lo, hi = blocks[..., byte], blocks[..., byte + 1]
        rows = np.stack([lo, hi], axis=-1).reshape(lead + (nb * BLOCK_ROWS, 2 * d))
        return rows
    vals = (blocks[..., byte] >> shift.astype(np.uint8)) if not _is8(codec) else blocks[..., byte]
    if _is8(codec):
        rows = vals
    else:
        vals = vals & 0xF
        rows = (vals[..., 0::2] | (vals[..., 1::2] << 4)).astype(np.uint8)
    return rows.reshape(lead + (nb * BLOCK_ROWS, row_bytes(codec, d)))


def unpack_scales(codec: str, role: str, d: int, blocks: np.ndarray) -> np.ndarray:
    """blocks uint16 [..., n_blocks, 32 * ng] -> [..., n_blocks * 32, ng]."""
    blocks = np.asarray(blocks)
    lead = blocks.shape[:-2]
    nb = blocks.shape[-2]
    idx = scale_positions(codec, role, d)
    ng = idx.shape[1]
    return blocks[..., idx].reshape(lead + (nb * BLOCK_ROWS, ng))


def plane_to_rows(plane, seq: int | None = None):
    """Reads a Plane back as (codes [S][H][capacity][row_bytes], scales uint16
    [S][H][capacity][ng]) in plain row order (host numpy arrays)."""
    d, cap = plane.head_dim, plane.capacity
    nb = cap // BLOCK_ROWS
    role = "k" if plane.role == 0 else "v"
    codes = plane.codes.cpu().numpy().reshape(plane.n_seqs, plane.n_kv_heads, nb, -1)
    scales = plane.scales.cpu().numpy().view(np.uint16).reshape(plane.n_seqs, plane.n_kv_heads, nb,
                                                                32 * n_scales(plane.codec, d))
    if seq is not None:
        codes, scales = codes[seq:seq + 1], scales[seq:seq + 1]
    return (unpack_codes(plane.codec, role, d, codes), unpack_scales(plane.codec, role, d, scales))
