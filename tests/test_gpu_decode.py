"""GPU decode-attention parity against the oracle (binary64 attention over the
oracle's own quantization of the same fp32 rows).

Bar: max|gpu - oracle| / max|oracle| <= 1e-3 over the outputs of one call
(per layer), the decode tolerance.  Covered: all
9 codec pairs, the f16 control codec (head_dim 64/128), head_dim 64/128/256, GQA 1..16, lengths 0, 1, ragged tails and
several tiles, device lengths beyond the host bound (cut to it) and negative
ones (empty), split-count sweeps, softmax invariants, and the tiny workload
configuration in full (the others, every head, in test_gpu_fullsize.py).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from block_quantized_kv_amd import Layer, kvq_attend_decode
from gpu_helpers import append_rows, rel_err

pytestmark = pytest.mark.gpu
TOL = 1e-3
CODECS = ["q8_0", "q4_0", "q4_g64"]


def _oracle_decode(kc, vc, q, k_rows, v_rows, length, scale, heads=None):
    """q [Hq][d] np; k_rows/v_rows np [n][H][d] fp32 -> oracle output."""
    kh = oracle.quant_dequant(kc, np.ascontiguousarray(k_rows.transpose(1, 0, 2)))
    vh = oracle.quant_dequant(vc, np.ascontiguousarray(v_rows.transpose(1, 0, 2)))
    return oracle.attend_decode(q, kh, vh, length, scale, heads=heads)


def _run_case(gpu, kc, vc, d, hq, hkv, lens, cap=None, seed=0, max_len=None, kv_scale=1.0):
    rng = np.random.default_rng(seed)
    S = len(lens)
    cap = cap or max(32, (max(lens) + 31) // 32 * 32)
    layer = Layer.create(kc, vc, d, hkv, S, cap, device=gpu)
    q = rng.standard_normal((S, hq, d)).astype(np.float32)
    ks, vs = [], []
    for s, n in enumerate(lens):
        k = (rng.standard_normal((cap, hkv, d)) * kv_scale).astype(np.float32)
        v = (rng.standard_normal((cap, hkv, d)) * kv_scale).astype(np.float32)
        append_rows(layer, torch.from_numpy(k).to(gpu), torch.from_numpy(v).to(gpu), s, 0)
        ks.append(k)
        vs.append(v)
    scale = 1.0 / np.sqrt(d)
    ml = max_len if max_len is not None else max(max(lens), 0)
    out = kvq_attend_decode(layer, torch.from_numpy(q).to(gpu),
                            torch.tensor(lens, dtype=torch.int64, device=gpu), ml, scale)
    out = out.cpu().numpy()
    for s, n in enumerate(lens):
        if n == 0:
            assert np.array_equal(out[s], np.zeros_like(out[s]))
            continue
        ref = _oracle_decode(kc, vc, q[s], ks[s], vs[s], n, scale)
        err = rel_err(out[s], ref)
        assert err <= TOL, (kc, vc, d, hq, hkv, n, err)
    return out


@pytest.mark.parametrize("kc", CODECS)
@pytest.mark.parametrize("vc", CODECS)
def test_codec_pairs_small(gpu, kc, vc):
    d = {"q8_0": 128, "q4_0": 64, "q4_g64": 256}[kc]
    _run_case(gpu, kc, vc, d, hq=8, hkv=2, lens=[1000, 33], seed=CODECS.index(kc) * 3 + CODECS.index(vc))


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("gqa", [1, 4, 6, 16])
def test_head_dims_and_gqa(gpu, d, gqa):
    _run_case(gpu, "q4_g64", "q4_0", d, hq=2 * gqa, hkv=2, lens=[257], seed=d + gqa)


@pytest.mark.parametrize("lens", [[1], [31, 32, 33], [0, 5, 64], [4097], [300, 0]])
def test_lengths_and_empty(gpu, lens):
    _run_case(gpu, "q8_0", "q4_g64", 128, hq=4, hkv=1, lens=lens, seed=sum(lens))


@pytest.mark.parametrize("max_len_factor", [1, 2, 8])
def test_split_sweep(gpu, max_len_factor):
    # max_len changes the split size and count; the result must not
    n = 3000
    _run_case(gpu, "q4_0", "q8_0", 128, hq=8, hkv=2, lens=[n], cap=n * 8 + 32,
              max_len=n * max_len_factor, seed=11)


@pytest.mark.parametrize("lens,max_len", [([5000], 3000), ([5000, 100, -3, 2999], 3000), ([-1], 64)])
def test_device_lengths_clamped_to_max_len(gpu, lens, max_len):
    """The call attends rows [0, min(seq_len[b], max_len)) of every sequence, a
    negative device length counting as 0: lengths past the host bound are cut
    to it, in the one-sequence grid and in the batched work list alike."""
    rng = np.random.default_rng(21)
    d, hq, hkv = 128, 8, 2
    S, cap = len(lens), 5024
    layer = Layer.create("q8_0", "q4_0", d, hkv, S, cap, device=gpu)
    q = rng.standard_normal((S, hq, d)).astype(np.float32)
    ks, vs = [], []
    for s in range(S):
        k = rng.standard_normal((cap, hkv, d)).astype(np.float32)
        v = rng.standard_normal((cap, hkv, d)).astype(np.float32)
        append_rows(layer, torch.from_numpy(k).to(gpu), torch.from_numpy(v).to(gpu), s, 0)
        ks.append(k)
        vs.append(v)
    scale = 1.0 / np.sqrt(d)
    out = kvq_attend_decode(layer, torch.from_numpy(q).to(gpu), torch.tensor(lens, dtype=torch.int64, device=gpu),
                            max_len, scale).cpu().numpy()
    for s, n in enumerate(lens):
        eff = min(max(n, 0), max_len)
        if eff == 0:
            assert np.array_equal(out[s], np.zeros_like(out[s]))
            continue
        ref = _oracle_decode("q8_0", "q4_0", q[s], ks[s], vs[s], eff, scale)
        assert rel_err(out[s], ref) <= TOL, (s, n, eff)


def test_large_and_small_magnitudes(gpu):
    _run_case(gpu, "q8_0", "q4_g64", 64, hq=4, hkv=1, lens=[500], kv_scale=1e-5, seed=3)
    _run_case(gpu, "q8_0", "q4_g64", 64, hq=4, hkv=1, lens=[500], kv_scale=300.0, seed=4)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("gqa", [1, 4, 16])
def test_f16_control_codec(gpu, d, gqa):
    # the f16 control: binary16 K and V through the same decode kernel
    _run_case(gpu, "f16", "f16", d, hq=2 * gqa, hkv=2, lens=[3001, 33, 0, 1], seed=d * 3 + gqa)


def test_f16_control_split_sweep_and_magnitudes(gpu):
    _run_case(gpu, "f16", "f16", 128, hq=8, hkv=2, lens=[3000], cap=24032, max_len=24000, seed=12)
    _run_case(gpu, "f16", "f16", 64, hq=4, hkv=1, lens=[500], kv_scale=1e-3, seed=13)
    _run_case(gpu, "f16", "f16", 64, hq=4, hkv=1, lens=[500], kv_scale=300.0, seed=14)


def test_f16_garbage_rows_past_length_are_ignored(gpu):
    """f16 planes have no scales to zero: binary16 NaN/Inf patterns in rows past
    the length (never appended) must not reach the output."""
    d, H, n = 128, 1, 45
    layer = Layer.create("f16", "f16", d, H, 1, 64, device=gpu)
    layer.k.codes.fill_(0xFF)  # 0xFFFF: NaN
    layer.v.codes.fill_(0x7C)  # 0x7C7C: NaN
    rng = np.random.default_rng(2)
    k = rng.standard_normal((n, H, d)).astype(np.float32)
    v = rng.standard_normal((n, H, d)).astype(np.float32)
    append_rows(layer, torch.from_numpy(k).to(gpu), torch.from_numpy(v).to(gpu), 0, 0)
    q = rng.standard_normal((1, 4, d)).astype(np.float32)
    out = kvq_attend_decode(layer, torch.from_numpy(q).to(gpu), torch.tensor([n], device=gpu), n,
                            0.1).cpu().numpy()
    ref = _oracle_decode("f16", "f16", q[0], k, v, n, 0.1)
    assert np.isfinite(out).all() and rel_err(out[0], ref) <= TOL


def test_invariants_constant_v_and_single_row(gpu):
    d, H, n = 128, 1, 700
    layer = Layer.create("q4_g64", "q8_0", d, H, 1, 704, device=gpu)
    rng = np.random.default_rng(9)
    k = rng.standard_normal((n, H, d)).astype(np.float32)
    row = np.round(rng.standard_normal(d) * 4).astype(np.float32)  # exactly representable codes
    row[0] = 127.0
    v = np.broadcast_to(row, (n, H, d)).copy()
    append_rows(layer, torch.from_numpy(k).to(gpu), torch.from_numpy(v).to(gpu), 0, 0)
    q = torch.randn(1, 4, d, device=gpu)
    v_hat = oracle.quant_dequant("q8_0", row[None])[0]   # what the cache holds
    out = kvq_attend_decode(layer, q, torch.tensor([n], device=gpu), n, 0.125).cpu().numpy()
    assert rel_err(out[0], np.broadcast_to(v_hat, (4, d))) <= TOL
    out1 = kvq_attend_decode(layer, q, torch.tensor([1], device=gpu), n, 0.125).cpu().numpy()
    assert rel_err(out1[0], np.broadcast_to(v_hat, (4, d))) <= TOL


def test_workspace_poison_does_not_leak(gpu):
    d, H, n = 128, 2, 2000
    layer = Layer.create("q8_0", "q4_0", d, H, 1, 2016, device=gpu)
    k = torch.randn(n, H, d, device=gpu)
    append_rows(layer, k, k, 0, 0)
    q = torch.randn(1, 8, d, device=gpu)
    lens = torch.tensor([n], device=gpu)
    from block_quantized_kv_amd import kvq_decode_workspace_bytes
    ws = torch.empty(kvq_decode_workspace_bytes(layer, 8, 1, n), dtype=torch.uint8, device=gpu)
    ws.view(torch.float32)[: ws.numel() // 4].fill_(float("nan"))
    a = kvq_attend_decode(layer, q, lens, n, 0.1, workspace=ws)
    b = kvq_attend_decode(layer, q, lens, n, 0.1)
    assert torch.isfinite(a).all() and torch.equal(a, b)
    c = kvq_attend_decode(layer, q, lens, n, 0.1, workspace=ws)  # reuse
    assert torch.equal(a, c)


def test_garbage_rows_past_length_are_ignored(gpu):
    """Rows past len_b inside the last block may hold anything (never appended):
    NaN/Inf scale bit patterns there must not reach the output."""
    d, H, n = 128, 1, 45
    layer = Layer.create("q8_0", "q4_0", d, H, 1, 64, device=gpu)
    layer.k.scales.fill_(0x7E00)  # binary16 NaN everywhere
    layer.v.scales.fill_(0x7C00)  # binary16 +inf everywhere
    layer.v.codes.fill_(0x3C)
    rng = np.random.default_rng(2)
    k = rng.standard_normal((n, H, d)).astype(np.float32)
    v = rng.standard_normal((n, H, d)).astype(np.float32)
    append_rows(layer, torch.from_numpy(k).to(gpu), torch.from_numpy(v).to(gpu), 0, 0)
    q = rng.standard_normal((1, 4, d)).astype(np.float32)
    out = kvq_attend_decode(layer, torch.from_numpy(q).to(gpu), torch.tensor([n], device=gpu), n,
                            0.1).cpu().numpy()
    ref = _oracle_decode("q8_0", "q4_0", q[0], k, v, n, 0.1)
    assert np.isfinite(out).all() and rel_err(out[0], ref) <= TOL


def test_graph_replay_matches_eager(gpu):
    """append + decode captured in a HIP graph: every replay equals the eager call
    (the library only enqueues kernels: no allocation, sync or memset)."""
    d, H, n = 256, 4, 4000
    layer = Layer.create("q4_g64", "q4_g64", d, H, 1, 4032, device=gpu)
    k = torch.randn(n, H, d, device=gpu)
    v = torch.randn(n, H, d, device=gpu)
    append_rows(layer, k[:-1], v[:-1], 0, 0)
    q = torch.randn(1, 24, d, device=gpu)
    lens = torch.tensor([n], device=gpu)
    from block_quantized_kv_amd import decode_workspace, kvq_append
    ws = decode_workspace(layer, 24, 1, n)
    sq = torch.zeros(1, dtype=torch.int32, device=gpu)
    pos = torch.tensor([n - 1], dtype=torch.int64, device=gpu)
    out = torch.empty_like(q)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        kvq_append(layer, k[-1:].contiguous(), v[-1:].contiguous(), sq, pos, stream=s)
        kvq_attend_decode(layer, q, lens, n, 0.0625, out=out, workspace=ws, stream=s)
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        kvq_append(layer, k[-1:].contiguous(), v[-1:].contiguous(), sq, pos, stream=s)
        kvq_attend_decode(layer, q, lens, n, 0.0625, out=out, workspace=ws, stream=s)
    for i in range(4):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), i
        kvq_attend_decode(layer, q, lens, n, 0.0625, workspace=ws)  # eager work between replays


# ---- the five workload configurations at full size ------------------------------

def _full_workload(gpu, cfg, layer_idx=0, append_last=False):
    kc, vc = cfg.layers[layer_idx]
    lens = workloads.seq_lengths(cfg, "cpu").tolist()
    layer = Layer.create(kc, vc, cfg.head_dim, cfg.n_kv_heads, cfg.n_seqs, cfg.capacity, device=gpu)
    q = workloads.queries(cfg, layer_idx, gpu)
    host_rows = []
    for s, n in enumerate(lens):
        k = workloads.kv_rows(cfg, layer_idx, s, "k", 0, n, gpu)
        v = workloads.kv_rows(cfg, layer_idx, s, "v", 0, n, gpu)
        if append_last:  # pre-fill n-1 rows, then the step's own one-row append
            append_rows(layer, k[:-1], v[:-1], s, 0)
            append_rows(layer, k[-1:], v[-1:], s, n - 1)
        else:
            append_rows(layer, k, v, s, 0)
        host_rows.append((k, v))
    out = kvq_attend_decode(layer, q, torch.tensor(lens, dtype=torch.int64, device=gpu),
                            max(lens), cfg.scale).cpu().numpy()
    qn = q.cpu().numpy()
    G = cfg.gqa
    worst = 0.0
    for s, n in enumerate(lens):
        for g in range(cfg.n_kv_heads):
            k, v = host_rows[s]
            kh = k[:, g:g + 1].cpu().numpy()
            vh = v[:, g:g + 1].cpu().numpy()
            heads = list(range(g * G, (g + 1) * G))
            ref = _oracle_decode(kc, vc, qn[s][heads], kh, vh, n, cfg.scale)
            worst = max(worst, rel_err(out[s][heads], ref))
    assert worst <= TOL, (cfg.name, layer_idx, worst)
    return worst


def test_tiny_decode_full(gpu):
    _full_workload(gpu, workloads.TINY)


# The 32K, 64K, 196K and batched configurations at full size, every head and
# layer, are in test_gpu_fullsize.py.
