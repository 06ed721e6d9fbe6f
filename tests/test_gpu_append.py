"""GPU quantize-on-append and dequant parity: codes and scales bit-exact
against the oracle (den_llama.cpp, "Results": quantizer byte-identical to the
CPU reference, dequant bit-identical), on every codec, both plane roles and
head_dim 64/128/256, with inputs that stress every rounding path; whole
aligned 32-row blocks (written word by word) beside scattered rows in one
call; one plane at a time (the other input absent)."""
import numpy as np
import pytest
import torch

import oracle
from block_quantized_kv_amd import Layer, kvq_append, kvq_dequant, layout

pytestmark = pytest.mark.gpu
CODECS = ["q8_0", "q4_0", "q4_g64"]


def _stress_rows(rng, n, H, d, codec):
    """fp32 [n][H][d] where every group is one of: N(0, sigma) with sigma over
    2^-24..2^12, exact ties on a power-of-two grid, all zeros, fp16-subnormal
    scales, scales above 65504 (saturation), a single non-zero value."""
    G, qmax = oracle.GROUP[codec], oracle.QMAX[codec]
    x = np.zeros((n, H, d // G, G), np.float32)
    kinds = rng.integers(0, 6, size=(n, H, d // G))
    for idx in np.ndindex(*kinds.shape):
        k = kinds[idx]
        if k == 0:
            x[idx] = rng.standard_normal(G) * 2.0 ** rng.uniform(-24, 12)
        elif k == 1:
            e = int(rng.integers(-10, 6))
            q = rng.integers(-qmax, qmax, size=G) + 0.5
            q[0] = qmax
            x[idx] = (q * 2.0 ** e).astype(np.float32)
        elif k == 2:
            pass
        elif k == 3:
            x[idx] = rng.standard_normal(G) * 2.0 ** rng.uniform(-30, -22)
        elif k == 4:
            x[idx] = rng.standard_normal(G) * (1e7 if codec == "q8_0" else 6e5)
        else:
            x[idx][rng.integers(G)] = rng.standard_normal() * 10
    return x.reshape(n, H, d)


@pytest.mark.parametrize("codec", CODECS)
@pytest.mark.parametrize("d", [64, 128, 256])
def test_append_bit_exact_scattered(gpu, codec, d):
    rng = np.random.default_rng(d * 7 + len(codec))
    H, S, cap, n = 3, 2, 128, 150
    # distinct (seq, pos) pairs, many sharing 32-row blocks (V nibble words)
    flat = rng.choice(S * cap, size=n, replace=False)
    seq, pos = flat // cap, flat % cap
    xk = _stress_rows(rng, n, H, d, codec)
    xv = _stress_rows(rng, n, H, d, codec)
    layer = Layer.create(codec, codec, d, H, S, cap, device=gpu)
    kvq_append(layer, torch.from_numpy(xk).to(gpu), torch.from_numpy(xv).to(gpu),
               torch.from_numpy(seq.astype(np.int32)).to(gpu),
               torch.from_numpy(pos.astype(np.int64)).to(gpu))
    for plane, x in ((layer.k, xk), (layer.v, xv)):
        codes, scales = layout.plane_to_rows(plane)
        want_c, want_s = oracle.quantize_rows(codec, x)                  # [n][H][...]
        assert np.array_equal(codes[seq, :, pos], want_c)
        assert np.array_equal(scales[seq, :, pos], want_s)
        untouched = np.ones((S, cap), bool)
        untouched[seq, pos] = False
        assert not codes.transpose(0, 2, 1, 3)[untouched].any()
        assert not scales.transpose(0, 2, 1, 3)[untouched].any()
        # dequant: bit-exact against the oracle's dequantization of its own codes
        want_hat = oracle.dequant_rows(codec, want_c, want_s, d)          # [n][H][d]
        for s in range(S):
            got = kvq_dequant(plane, s, 0, cap).cpu().numpy()              # [H][cap][d]
            m = seq == s
            assert np.array_equal(got[:, pos[m]].transpose(1, 0, 2).view(np.uint32),
                                  want_hat[m].view(np.uint32))


@pytest.mark.parametrize("kc,vc,d", [("q8_0", "q4_0", 128), ("q4_g64", "q4_g64", 256), ("q4_0", "q8_0", 64)])
def test_append_whole_blocks_and_others_in_one_call(gpu, kc, vc, d):
    # one call whose 32-token groups are: an aligned block of sequence 0, a
    # block-sized run starting mid-block, an aligned block of sequence 1,
    # 32 tokens that straddle two sequences, and a ragged tail of 7: whole V
    # blocks are written word by word, the rest value by value
    rng = np.random.default_rng(d + len(kc) * 10 + len(vc))
    H, S, cap = 2, 2, 256
    seq = np.concatenate([np.zeros(32), np.zeros(32), np.ones(32), np.r_[np.zeros(16), np.ones(16)],
                          np.ones(7)]).astype(np.int32)
    pos = np.concatenate([np.arange(64, 96), np.arange(144, 176), np.arange(32, 64),
                          np.r_[np.arange(200, 216), np.arange(100, 116)], np.arange(240, 247)]).astype(np.int64)
    n = len(seq)
    xk = _stress_rows(rng, n, H, d, kc)
    xv = _stress_rows(rng, n, H, d, vc)
    layer = Layer.create(kc, vc, d, H, S, cap, device=gpu)
    kvq_append(layer, torch.from_numpy(xk).to(gpu), torch.from_numpy(xv).to(gpu),
               torch.from_numpy(seq).to(gpu), torch.from_numpy(pos).to(gpu))
    for plane, x, codec in ((layer.k, xk, kc), (layer.v, xv, vc)):
        codes, scales = layout.plane_to_rows(plane)
        want_c, want_s = oracle.quantize_rows(codec, x)
        assert np.array_equal(codes[seq, :, pos], want_c), codec
        assert np.array_equal(scales[seq, :, pos], want_s), codec
        untouched = np.ones((S, cap), bool)
        untouched[seq, pos] = False
        assert not codes.transpose(0, 2, 1, 3)[untouched].any()
        assert not scales.transpose(0, 2, 1, 3)[untouched].any()


@pytest.mark.parametrize("codec", CODECS)
def test_append_overwrites_rows(gpu, codec):
    # a second append to the same positions replaces every code and scale
    rng = np.random.default_rng(5)
    H, d, cap = 2, 128, 64
    layer = Layer.create(codec, codec, d, H, 1, cap, device=gpu)
    pos = torch.arange(0, 64, dtype=torch.int64, device=gpu)
    sq = torch.zeros(64, dtype=torch.int32, device=gpu)
    for trial in range(2):
        x = _stress_rows(rng, 64, H, d, codec)
        xt = torch.from_numpy(x).to(gpu)
        kvq_append(layer, xt, xt, sq, pos)
        for plane in (layer.k, layer.v):
            codes, scales = layout.plane_to_rows(plane)
            wc, ws = oracle.quantize_rows(codec, x)
            assert np.array_equal(codes[0].transpose(1, 0, 2), wc)
            assert np.array_equal(scales[0].transpose(1, 0, 2), ws)


@pytest.mark.parametrize("kc,vc,d", [("q8_0", "q4_0", 128), ("q4_g64", "q4_g64", 256)])
def test_append_one_plane_at_a_time(gpu, kc, vc, d):
    # k only, then v only (a whole aligned block and a ragged tail of 9 rows):
    # the plane without input is left as it was
    rng = np.random.default_rng(d + 3)
    H, cap = 2, 64
    n = 41
    pos = np.arange(n, dtype=np.int64)
    seq = np.zeros(n, np.int32)
    xk = _stress_rows(rng, n, H, d, kc)
    xv = _stress_rows(rng, n, H, d, vc)
    layer = Layer.create(kc, vc, d, H, 1, cap, device=gpu)
    sq, ps = torch.from_numpy(seq).to(gpu), torch.from_numpy(pos).to(gpu)
    kvq_append(layer, torch.from_numpy(xk).to(gpu), None, sq, ps)
    codes_v, scales_v = layout.plane_to_rows(layer.v)
    assert not codes_v.any() and not scales_v.any()
    kvq_append(layer, None, torch.from_numpy(xv).to(gpu), sq, ps)
    for plane, x, codec in ((layer.k, xk, kc), (layer.v, xv, vc)):
        codes, scales = layout.plane_to_rows(plane)
        want_c, want_s = oracle.quantize_rows(codec, x)
        assert np.array_equal(codes[seq, :, pos], want_c), codec
        assert np.array_equal(scales[seq, :, pos], want_s), codec
        assert not codes[0, :, n:].any() and not scales[0, :, n:].any()


def test_append_out_of_range_positions_flagged(gpu):
    H, d, cap = 1, 64, 64
    layer = Layer.create("q4_0", "q4_g64", d, H, 1, cap, device=gpu)
    x = torch.ones(3, H, d, device=gpu)
    status = torch.zeros(1, dtype=torch.int32, device=gpu)
    pos = torch.tensor([5, 64, -1], dtype=torch.int64, device=gpu)
    sq = torch.tensor([0, 0, 0], dtype=torch.int32, device=gpu)
    kvq_append(layer, x, x, sq, pos, dev_status=status)
    assert int(status.item()) == 3  # KVQ_ERANGE
    codes, _ = layout.plane_to_rows(layer.k)
    assert codes[0, 0, 5].any()
    status.zero_()
    kvq_append(layer, x[:1], x[:1], sq[:1], pos[:1], dev_status=status)
    assert int(status.item()) == 0
    with pytest.raises(ValueError):
        kvq_append(layer, x, x, sq, pos[:2])  # size mismatch caught on the host, nothing launched


def test_append_full_workload_plane_bit_exact(gpu):
    """The 64K-context Q4_G64 plane of the decode workload, checked whole."""
    import workloads
    cfg = workloads.DECODE_64K
    layer = Layer.create("q4_g64", "q4_g64", cfg.head_dim, cfg.n_kv_heads, 1, cfg.capacity, device=gpu)
    k = workloads.kv_rows(cfg, 0, 0, "k", 0, cfg.ctx, gpu)
    v = workloads.kv_rows(cfg, 0, 0, "v", 0, cfg.ctx, gpu)
    from gpu_helpers import append_rows
    append_rows(layer, k, v, 0, 0)
    for plane, x in ((layer.k, k), (layer.v, v)):
        codes, scales = layout.plane_to_rows(plane)
        xn = x.cpu().numpy().transpose(1, 0, 2)                          # [H][n][d]
        wc, ws = oracle.quantize_rows("q4_g64", xn)
        assert np.array_equal(codes[0], wc)
        assert np.array_equal(scales[0], ws)


def _f16_rows(rng, n, H, d):
    """fp32 rows for the f16 control codec: magnitudes over 1e-8..1e5, with
    per-row values at a binary16 tie, beyond the range (saturation) and in the
    binary16 subnormal range."""
    x = rng.standard_normal((n, H, d)) * 10.0 ** rng.uniform(-8, 5, (n, H, 1))
    x[..., 0] = 1 + 2.0 ** -11
    x[..., 1] = 7e4
    x[..., 2] = -1e6
    x[..., 3] = 2.0 ** -25
    x[..., 4] = 3 * 2.0 ** -26
    return x.astype(np.float32)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_append_f16_control_bit_exact(gpu, d):
    """The f16 control codec: every stored value is the oracle's (binary16
    nearest-even, saturated), in both plane roles; nothing else written;
    dequant returns it exactly."""
    rng = np.random.default_rng(d + 16)
    H, S, cap, n = 3, 2, 96, 110
    flat = rng.choice(S * cap, size=n, replace=False)
    seq, pos = flat // cap, flat % cap
    xk, xv = _f16_rows(rng, n, H, d), _f16_rows(rng, n, H, d)
    layer = Layer.create("f16", "f16", d, H, S, cap, device=gpu)
    kvq_append(layer, torch.from_numpy(xk).to(gpu), torch.from_numpy(xv).to(gpu),
               torch.from_numpy(seq.astype(np.int32)).to(gpu), torch.from_numpy(pos.astype(np.int64)).to(gpu))
    for plane, x in ((layer.k, xk), (layer.v, xv)):
        codes, _ = layout.plane_to_rows(plane)
        want_c, want_s = oracle.quantize_rows("f16", x)
        assert np.array_equal(codes[seq, :, pos], want_c)
        untouched = np.ones((S, cap), bool)
        untouched[seq, pos] = False
        assert not codes.transpose(0, 2, 1, 3)[untouched].any()
        want_hat = oracle.dequant_rows("f16", want_c, want_s, d)
        for s in range(S):
            got = kvq_dequant(plane, s, 0, cap).cpu().numpy()
            m = seq == s
            assert np.array_equal(got[:, pos[m]].transpose(1, 0, 2).view(np.uint32), want_hat[m].view(np.uint32))
