"""Pins for the oracle quantizer / dequantizer.

What fixes the expected values (none of it is the oracle itself):
  * hand-worked blocks in tests/golden/quant_blocks.txt, each derived by hand
    from the codec definitions (den_llama.cpp, section "What this fork is":
    Q4_G64 = signed INT4 + one FP16 scale per 64 values, 4.25 bits/value;
    q8_0 / q4_0, named on the same page, take the same rule at 32 values per
    group);
  * the 4.25 / 4.5 / 8.5 bits-per-value size arithmetic;
  * brute force: the stored scale is the binary16 nearest to amax/Qmax (searched
    over all 65536 patterns) and every code is the integer in range nearest to
    x/dq (searched over all candidates), ties to even;
  * invariants: round-trip error at most dq/2 (plus the binary32 quotient
    rounding), idempotence, sign symmetry, power-of-two scaling, exact grids,
    exact dequantization.
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quant_blocks.txt")
CODECS = ["q8_0", "q4_0", "q4_g64"]


def _parse_golden():
    blocks, cur = [], {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            if cur:
                blocks.append(cur)
                cur = {}
            continue
        key, _, rest = line.partition(" ")
        cur[key] = rest
    if cur:
        blocks.append(cur)
    return [b for b in blocks if "codec" in b]


def _num(tok: str) -> float:
    return float.fromhex(tok) if "0x" in tok.lower() else float(tok)


@pytest.mark.parametrize("blk", _parse_golden(), ids=lambda b: b["codec"] + ":" + b["x"][:24])
def test_golden_blocks(blk):
    codec = blk["codec"]
    G = oracle.GROUP[codec]
    vals = [_num(t) for t in blk["x"].split()]
    x = np.zeros(G, np.float32)
    x[: len(vals)] = vals
    scale, q = oracle.quantize_group(codec, x)
    assert scale == int(blk["scale"], 16), hex(scale)
    codes = [int(t) for t in blk["codes"].split()]
    want = np.zeros(G, np.int32)
    want[: len(codes)] = codes
    assert np.array_equal(q, want), q[: len(codes)]
    if "bytes" in blk:
        c, s = oracle.quantize_rows(codec, x[None])
        wb = bytes(int(t, 16) for t in blk["bytes"].split())
        assert c[0, : len(wb)].tobytes() == wb, c[0, : len(wb)].tobytes().hex()
        assert s[0, 0] == int(blk["scale"], 16)


def test_golden_block_F_identity_grid():
    # x_i = (i mod 15) - 7: amax 7, scale 1, codes equal x exactly, error 0.
    x = (np.arange(64) % 15 - 7).astype(np.float32)
    scale, q = oracle.quantize_group("q4_g64", x)
    assert scale == 0x3C00
    assert np.array_equal(q, x.astype(np.int32))
    assert np.array_equal(oracle.quant_dequant("q4_g64", x[None])[0], x)


@pytest.mark.parametrize("codec,bpv", [("q4_g64", 4.25), ("q4_0", 4.5), ("q8_0", 8.5)])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_bits_per_value(codec, bpv, d):
    # den_llama.cpp, "What this fork is": Q4_G64 is 4.25 bits per value.
    x = np.ones((3, d), np.float32)
    c, s = oracle.quantize_rows(codec, x)
    assert (c.shape[1] + 2 * s.shape[1]) * 8 / d == bpv


def _all_f16_values():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = h.view(np.float16).astype(np.float64)
    ok = np.isfinite(v) & (v >= 0)
    return h[ok], v[ok]


_F16_BITS, _F16_VALS = _all_f16_values()


def _nearest_f16_bits(t: float) -> int:
    """Brute force: the binary16 pattern nearest to t >= 0, ties to even fraction."""
    t = min(t, 65504.0)
    dist = np.abs(_F16_VALS - t)
    best = np.nonzero(dist == dist.min())[0]
    cands = _F16_BITS[best]
    if len(cands) > 1:
        even = [c for c in cands if (c & 1) == 0]
        cands = even or cands
    return int(min(cands))


def _nearest_code(t: float, qmax: int) -> int:
    """Brute force: the integer in [-qmax-1, qmax] nearest to t, ties to even."""
    cands = np.arange(-qmax - 1, qmax + 1)
    dist = np.abs(cands - t)
    best = cands[dist == dist.min()]
    if len(best) > 1:
        best = best[best % 2 == 0]
    return int(best[0])


@pytest.mark.parametrize("codec", CODECS)
def test_brute_force_scale_and_codes(codec):
    rng = np.random.default_rng(1234)
    G, qmax = oracle.GROUP[codec], oracle.QMAX[codec]
    for trial in range(60):
        sigma = 2.0 ** rng.uniform(-26, 12)
        x = (rng.standard_normal(G) * sigma).astype(np.float32)
        if trial % 7 == 0:  # plant exact ties on the grid of the expected scale
            x[: G // 2] = (np.round(x[: G // 2] / sigma * 4) / 4 * sigma).astype(np.float32)
        scale, q = oracle.quantize_group(codec, x)
        amax = float(np.max(np.abs(x)))
        d32 = np.float32(np.float32(amax) / np.float32(qmax))
        assert scale == _nearest_f16_bits(float(d32))
        dq = float(np.uint16(scale).view(np.float16))
        for i in range(G):
            if dq == 0.0:
                assert q[i] == 0
            else:
                t = float(np.float32(x[i]) / np.float32(dq))  # binary32 quotient
                assert q[i] == _nearest_code(t, qmax), (trial, i, x[i], dq, t, q[i])


def _rand_rows(rng, n, d, lo=-6, hi=6):
    sig = 2.0 ** rng.uniform(lo, hi, size=(n, 1))
    return (rng.standard_normal((n, d)) * sig).astype(np.float32)


@pytest.mark.parametrize("codec", CODECS)
def test_round_trip_bound(codec):
    rng = np.random.default_rng(7)
    d = 256
    x = _rand_rows(rng, 2000, d)
    c, s = oracle.quantize_rows(codec, x)
    xh = oracle.dequant_rows(codec, c, s, d)
    G = oracle.GROUP[codec]
    dq = np.repeat(s.view(np.float16).astype(np.float64), G, axis=1)
    err = np.abs(x.astype(np.float64) - xh.astype(np.float64))
    assert np.all(err <= dq / 2 + np.abs(x) * 2.0 ** -23)


@pytest.mark.parametrize("codec", CODECS)
def test_idempotence_and_dequant_exact(codec):
    rng = np.random.default_rng(8)
    d = 128
    x = _rand_rows(rng, 500, d)
    c, s = oracle.quantize_rows(codec, x)
    xh = oracle.dequant_rows(codec, c, s, d)
    # dequant exact: equals the binary64 product of code and scale
    G = oracle.GROUP[codec]
    qv = _codes_int(codec, c, d).astype(np.float64)
    dq = np.repeat(s.view(np.float16).astype(np.float64), G, axis=1)
    assert np.array_equal(xh.astype(np.float64), qv * dq)
    # re-quantizing the dequantized values reproduces codes and scales exactly
    # whenever a group's largest code reaches +-Qmax
    c2, s2 = oracle.quantize_rows(codec, xh)
    qmax = oracle.QMAX[codec]
    full = np.abs(qv).reshape(500, d // G, G).max(-1) == qmax
    assert np.array_equal(s2[full], s[full])
    q1 = qv.reshape(500, d // G, G)[full]
    q2 = _codes_int(codec, c2, d).reshape(500, d // G, G)[full]
    assert np.array_equal(q1, q2)


def _codes_int(codec, c, d):
    """Decode stored bytes to integer codes (test-side restatement of the storage)."""
    if codec == "q8_0":
        return c.view(np.int8).astype(np.int32)
    lo = (c & 0xF).astype(np.int32)
    hi = (c >> 4).astype(np.int32)
    nib = np.stack([lo, hi], axis=-1).reshape(c.shape[0], d)
    return nib - 8 if codec == "q4_0" else np.where(nib >= 8, nib - 16, nib)


@pytest.mark.parametrize("codec", CODECS)
def test_sign_symmetry(codec):
    rng = np.random.default_rng(9)
    d = 64
    x = _rand_rows(rng, 300, d)
    c1, s1 = oracle.quantize_rows(codec, x)
    c2, s2 = oracle.quantize_rows(codec, -x)
    assert np.array_equal(s1, s2)
    q1, q2 = _codes_int(codec, c1, d), _codes_int(codec, c2, d)
    assert np.array_equal(q1, -q2)
    if codec == "q4_0":  # stored nibble c' = 16 - c
        n1 = q1 + 8
        n2 = q2 + 8
        assert np.array_equal(n2, 16 - n1)


@pytest.mark.parametrize("codec", CODECS)
@pytest.mark.parametrize("k", [-5, -1, 1, 4])
def test_power_of_two_scaling(codec, k):
    rng = np.random.default_rng(10 + k)
    d = 64
    x = _rand_rows(rng, 300, d, lo=-2, hi=2)
    c1, s1 = oracle.quantize_rows(codec, x)
    c2, s2 = oracle.quantize_rows(codec, (x * np.float32(2.0 ** k)).astype(np.float32))
    assert np.array_equal(c1, c2)
    assert np.array_equal(s2.view(np.float16).astype(np.float64),
                          s1.view(np.float16).astype(np.float64) * 2.0 ** k)


@pytest.mark.parametrize("codec", CODECS)
def test_on_grid_inputs_exact(codec):
    rng = np.random.default_rng(11)
    G, qmax = oracle.GROUP[codec], oracle.QMAX[codec]
    d = 128
    q = rng.integers(-qmax, qmax + 1, size=(200, d))
    q[:, ::G] = qmax  # every group reaches +Qmax, so the scale is exactly dq
    dq = 2.0 ** rng.integers(-10, 4, size=(200, d // G))
    x = (q * np.repeat(dq, G, axis=1)).astype(np.float32)
    c, s = oracle.quantize_rows(codec, x)
    assert np.array_equal(oracle.dequant_rows(codec, c, s, d), x)


def test_nonfinite_input_rejected():
    x = np.zeros(32, np.float32)
    x[3] = np.nan
    with pytest.raises(ValueError):
        oracle.quantize_group("q8_0", x)


# ---- the f16 control codec ---------------------------------------------------------

def _f16_inputs():
    rng = np.random.default_rng(16)
    x = rng.standard_normal(4096) * 10.0 ** rng.uniform(-9, 6, 4096)
    one = 1.0
    specials = [0.0, -0.0, 1.0, -1.0, 65504.0, -65504.0, 65519.99, 65520.0, -65520.0, 1e6, -3e38,
                6.1e-5, 2.0 ** -14, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -26,
                one + 2.0 ** -11, one + 3 * 2.0 ** -11, -(one + 2.0 ** -11), 2049.0, 2051.0, 1e-8]
    return np.concatenate([x, specials, np.zeros(64 - (4096 + len(specials)) % 64)]).astype(np.float32)


def test_f16_codec_is_the_binary16_cast_with_saturation():
    """The f16 control codec stores each value as torch's binary16 cast (a
    library routine, round to nearest even) of the value clamped to +-65504,
    little-endian, with no scales; dequantization returns that binary16 value."""
    import torch
    x = _f16_inputs()
    codes, scales = oracle.quantize_rows("f16", x.reshape(-1, 64))
    assert codes.shape == (x.size // 64, 128) and scales.shape == (x.size // 64, 0)
    bits = codes.reshape(-1, 2)
    got = bits[:, 0].astype(np.uint16) | (bits[:, 1].astype(np.uint16) << 8)
    want = torch.from_numpy(np.clip(x, -65504, 65504)).half().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
    back = oracle.dequant_rows("f16", codes, scales, 64).reshape(-1)
    assert np.array_equal(back, want.view(np.float16).astype(np.float32))
    # round-trip error at most half a binary16 unit in the last place inside the range
    inside = np.abs(x) < 65504
    ulp = np.spacing(np.abs(back[inside]).astype(np.float16)).astype(np.float64)
    assert (np.abs(back[inside].astype(np.float64) - x[inside]) <= ulp / 2).all()
    assert oracle.row_code_bytes("f16", 128) == 256


def test_f16_codec_rejects_non_finite():
    x = np.zeros(64, np.float32)
    x[3] = np.inf
    with pytest.raises(ValueError):
        oracle.quantize_rows("f16", x)
