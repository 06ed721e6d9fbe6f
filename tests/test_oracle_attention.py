"""Pins for the oracle's binary64 attention (decode and chunked prefill).

Expected values come from a library routine (torch's scaled_dot_product_attention
in float64 on the CPU, with GQA expanded by repeat_interleave and an explicit
causal mask offset by the prefix length) and from softmax identities that hold
for any correct implementation: constant V, a single row, equal keys, zero
scale, GQA-shared queries, row permutation, a dominant score, and the
log-sum-exp merge of any row partition (the identity the split-K GPU kernels
rely on).
"""
import numpy as np
import pytest
import torch

import oracle


def _sdpa_decode(q, k, v, length, scale):
    hq, d = q.shape
    hkv = k.shape[0]
    g = hq // hkv
    qt = torch.from_numpy(q.astype(np.float64))[:, None, :]            # [Hq,1,d]
    kt = torch.from_numpy(k[:, :length].astype(np.float64)).repeat_interleave(g, 0)
    vt = torch.from_numpy(v[:, :length].astype(np.float64)).repeat_interleave(g, 0)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    return o[:, 0].numpy()


def _sdpa_prefill(q, k, v, P, scale):
    T, hq, d = q.shape
    hkv = k.shape[0]
    g = hq // hkv
    qt = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)         # [Hq,T,d]
    kt = torch.from_numpy(k[:, : P + T].astype(np.float64)).repeat_interleave(g, 0)
    vt = torch.from_numpy(v[:, : P + T].astype(np.float64)).repeat_interleave(g, 0)
    t = torch.arange(T)[:, None]
    j = torch.arange(P + T)[None, :]
    mask = j <= P + t                                                   # token t sees rows <= P+t
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return o.permute(1, 0, 2).numpy()


def _rel(a, b):
    return np.abs(a.astype(np.float64) - b).max() / np.abs(b).max()


@pytest.mark.parametrize("hq,hkv,d,n", [(4, 1, 64, 256), (8, 2, 128, 300), (6, 1, 256, 97),
                                        (32, 8, 128, 40)])
def test_decode_matches_sdpa(hq, hkv, d, n):
    rng = np.random.default_rng(hq * 1000 + n)
    q = rng.standard_normal((hq, d)).astype(np.float32)
    k = rng.standard_normal((hkv, n + 5, d)).astype(np.float32)
    v = rng.standard_normal((hkv, n + 5, d)).astype(np.float32)
    scale = 1 / np.sqrt(d)
    out = oracle.attend_decode(q, k, v, n, scale)
    ref = _sdpa_decode(q, k, v, n, scale)
    assert _rel(out, ref) < 1e-6  # output is rounded to binary32 once


@pytest.mark.parametrize("hq,hkv,d,P,T", [(4, 2, 64, 64, 16), (8, 2, 128, 0, 33), (4, 1, 64, 5, 7)])
def test_prefill_matches_sdpa(hq, hkv, d, P, T):
    rng = np.random.default_rng(P * 31 + T)
    q = rng.standard_normal((T, hq, d)).astype(np.float32)
    k = rng.standard_normal((hkv, P + T, d)).astype(np.float32)
    v = rng.standard_normal((hkv, P + T, d)).astype(np.float32)
    scale = 1 / np.sqrt(d)
    out = oracle.attend_prefill(q, k, v, P, scale)
    ref = _sdpa_prefill(q, k, v, P, scale)
    assert _rel(out, ref) < 1e-6


def test_prefill_token_is_decode_over_its_prefix():
    rng = np.random.default_rng(3)
    hq, hkv, d, P, T = 4, 2, 64, 20, 9
    q = rng.standard_normal((T, hq, d)).astype(np.float32)
    k = rng.standard_normal((hkv, P + T, d)).astype(np.float32)
    v = rng.standard_normal((hkv, P + T, d)).astype(np.float32)
    full = oracle.attend_prefill(q, k, v, P, 0.125)
    for t in range(T):
        dec = oracle.attend_decode(q[t], k, v, P + t + 1, 0.125)
        assert np.array_equal(full[t], dec)
    sel = oracle.attend_prefill(q, k, v, P, 0.125, tokens=[3, 8, 0], heads=[1, 3, 2])
    assert np.array_equal(sel, np.stack([full[3, 1], full[8, 3], full[0, 2]]))


def test_constant_v_returns_v():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((4, 64)).astype(np.float32)
    k = rng.standard_normal((1, 256, 64)).astype(np.float32)
    row = rng.standard_normal(64).astype(np.float32)
    v = np.broadcast_to(row, (1, 256, 64)).copy()
    out = oracle.attend_decode(q, k, v, 256, 0.125)
    assert np.allclose(out, row[None], rtol=0, atol=1e-6 * np.abs(row).max())


def test_single_row_returns_its_v():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((4, 64)).astype(np.float32)
    k = rng.standard_normal((1, 8, 64)).astype(np.float32)
    v = rng.standard_normal((1, 8, 64)).astype(np.float32)
    out = oracle.attend_decode(q, k, v, 1, 0.125)
    assert np.array_equal(out, np.broadcast_to(v[0, 0], out.shape))


def test_equal_keys_or_zero_scale_give_mean_of_v():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((4, 64)).astype(np.float32)
    k = np.broadcast_to(rng.standard_normal(64).astype(np.float32), (1, 100, 64)).copy()
    v = rng.standard_normal((1, 100, 64)).astype(np.float32)
    mean = v[0].astype(np.float64).mean(0)
    assert np.allclose(oracle.attend_decode(q, k, v, 100, 0.125), mean[None], rtol=0, atol=1e-6)
    k2 = rng.standard_normal((1, 100, 64)).astype(np.float32)
    assert np.allclose(oracle.attend_decode(q, k2, v, 100, 0.0), mean[None], rtol=0, atol=1e-6)


def test_gqa_mapping_contiguous_groups():
    # q-heads 0..G-1 read kv-head 0, G..2G-1 read kv-head 1, ...
    rng = np.random.default_rng(7)
    hq, hkv, d, n = 8, 2, 64, 50
    base = rng.standard_normal(d).astype(np.float32)
    q = np.broadcast_to(base, (hq, d)).copy()
    k = rng.standard_normal((hkv, n, d)).astype(np.float32)
    v = rng.standard_normal((hkv, n, d)).astype(np.float32)
    out = oracle.attend_decode(q, k, v, n, 0.125)
    for h in range(hq):
        assert np.array_equal(out[h], out[(h // 4) * 4])
    assert not np.allclose(out[0], out[4])
    solo = oracle.attend_decode(q[:4], k[1:2], v[1:2], n, 0.125)
    assert np.array_equal(out[4:], solo)


def test_row_permutation_invariance():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((4, 64)).astype(np.float32)
    k = rng.standard_normal((1, 200, 64)).astype(np.float32)
    v = rng.standard_normal((1, 200, 64)).astype(np.float32)
    perm = rng.permutation(200)
    a = oracle.attend_decode(q, k, v, 200, 0.125)
    b = oracle.attend_decode(q, k[:, perm], v[:, perm], 200, 0.125)
    assert _rel(a, b) < 1e-6


def test_dominant_score_selects_its_row():
    rng = np.random.default_rng(9)
    d = 64
    q = np.zeros((1, d), np.float32)
    q[0, 0] = 1.0
    k = rng.standard_normal((1, 64, d)).astype(np.float32) * 0.1
    k[0, 17, 0] = 1000.0  # score margin >= 100 over every other row
    v = rng.standard_normal((1, 64, d)).astype(np.float32)
    out = oracle.attend_decode(q, k, v, 64, 1.0)
    assert np.allclose(out[0], v[0, 17], rtol=0, atol=1e-30 + 1e-40)


def test_empty_sequence_is_zero():
    q = np.ones((4, 64), np.float32)
    k = np.ones((1, 8, 64), np.float32)
    assert np.array_equal(oracle.attend_decode(q, k, k, 0, 0.125), np.zeros((4, 64), np.float32))


@pytest.mark.parametrize("cuts", [[0, 300], [0, 1, 300], [0, 64, 65, 200, 300], [0, 17, 34, 290, 300]])
def test_lse_merge_of_any_partition(cuts):
    """Split rows into chunks, attend each chunk, merge with
    out = sum_s exp(lse_s - LSE) out_s: equals attending all rows."""
    rng = np.random.default_rng(len(cuts))
    d = 128
    q = rng.standard_normal((2, d)).astype(np.float32)
    k = rng.standard_normal((1, 300, d)).astype(np.float32)
    v = rng.standard_normal((1, 300, d)).astype(np.float32)
    scale = 1 / np.sqrt(d)
    whole = oracle.attend_decode(q, k, v, 300, scale).astype(np.float64)
    s = (q.astype(np.float64) @ k[0].astype(np.float64).T) * scale           # [2,300]
    outs, lses = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        outs.append(oracle.attend_decode(q, k[:, a:b], v[:, a:b], b - a, scale).astype(np.float64))
        m = s[:, a:b].max(1)
        lses.append(m + np.log(np.exp(s[:, a:b] - m[:, None]).sum(1)))
    lse = np.stack(lses)                                                    # [S,2]
    L = lse.max(0) + np.log(np.exp(lse - lse.max(0)).sum(0))
    merged = sum(np.exp(lse[i] - L)[:, None] * outs[i] for i in range(len(outs)))
    assert np.abs(merged - whole).max() / np.abs(whole).max() < 1e-6
