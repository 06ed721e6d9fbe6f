"""Pins for the oracle's own binary16 conversion (written from the IEEE format
definition) against library conversions.

The quantizer's scale is stored as a binary16 rounded to nearest even (the
Q4_G64 codec of den_llama.cpp, section "What this fork is": "one FP16 scale per
64 values"), so the oracle's conversion must agree with an independent one on
every rounding-relevant input.
"""
import numpy as np
import torch

import oracle


def _lib_f16_bits(x: np.ndarray) -> np.ndarray:
    # torch's CPU float->half cast (round to nearest even, subnormals kept).
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float16).view(torch.int16).numpy().view(np.uint16)


def _compare(bits: np.ndarray) -> None:
    x = bits.view(np.float32)
    got = oracle.f32_to_f16_bits_array(x)
    want = _lib_f16_bits(x)
    nan = np.isnan(x)
    bad = np.nonzero((got != want) & ~nan)[0]
    assert bad.size == 0, [(hex(int(bits[i])), hex(int(got[i])), hex(int(want[i]))) for i in bad[:5]]
    # NaN must stay NaN (payload is not specified).
    g = got[nan]
    assert np.all(((g & 0x7C00) == 0x7C00) & ((g & 0x03FF) != 0))


def test_f16_normal_range_rounding_positions():
    # Normal results round at binary32 fraction bit 13: enumerate every value of
    # bits [13, 32) combined with the low-13-bit patterns that decide rounding
    # (exact, just below/at/above the half, and a few arbitrary ones).
    low = np.array([0x0000, 0x0001, 0x0FFF, 0x1000, 0x1001, 0x1FFF, 0x0800, 0x17FF,
                    0x0123, 0x0ABC, 0x1357, 0x1ACE], dtype=np.uint32)
    high = (np.arange(1 << 19, dtype=np.uint32) << 13)
    bits = (high[:, None] | low[None, :]).ravel()
    _compare(bits)


def test_f16_subnormal_and_overflow_exponents_exhaustive():
    # Every binary32 pattern whose exponent lands in the binary16 subnormal
    # range or at the overflow boundary (both signs): here the rounding
    # position moves with the exponent, so all fractions are checked.
    frac = np.arange(1 << 23, dtype=np.uint32)
    for e32 in list(range(100, 114)) + [142, 143]:
        for sign in (0, 1):
            bits = (np.uint32(sign << 31) | np.uint32(e32 << 23) | frac)
            _compare(bits)


def test_f16_special_values():
    for x, h in [(0.0, 0x0000), (-0.0, 0x8000), (1.0, 0x3C00), (-2.0, 0xC000),
                 (65504.0, 0x7BFF), (65519.996, 0x7BFF), (65520.0, 0x7C00),
                 (float("inf"), 0x7C00), (float("-inf"), 0xFC00),
                 (2.0 ** -24, 0x0001), (2.0 ** -25, 0x0000), (2.0 ** -25 * 1.5, 0x0001),
                 (2.0 ** -14, 0x0400), (1e-45, 0x0000)]:
        assert oracle.f32_to_f16_bits(x) == h, (x, hex(oracle.f32_to_f16_bits(x)), hex(h))


def test_f16_to_f32_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    want = bits.view(np.float16).astype(np.float32)
    got = np.array([oracle.f16_bits_to_f32(int(b)) for b in bits], dtype=np.float32)
    nan = np.isnan(want)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))
    assert np.all(np.isnan(got[nan]))
