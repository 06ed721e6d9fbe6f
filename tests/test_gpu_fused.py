"""GPU parity of the fused append + decode calls.

kvq_append_attend_decode(_mq) must leave the cache byte for byte as
kvq_append does (every byte of both planes is compared, so nothing outside
the new rows may change), and return what kvq_attend_decode(_mq) returns on
that cache: to 5e-4 of max|out|, not bit for bit, because the waves of a
split take blocks in whatever order they get them, and the binary16
probabilities are rounded relative to a running maximum that depends on that
order (2^-11 relative); and within the decode bar, 1e-3 of max|oracle|, of
binary64 attention over the oracle's own quantization, new rows included.

Covered: every codec pair; head_dim 64, 128 and 256; the new row at the start
of a block, at the end of a block, as the last row of a split and as the
first row of a split of its own; a sequence of length 1; a sequence of
length 0 (nothing written, output 0) among others; two and three new rows
straddling a block and a split boundary; the new row deep in a long split
(its block waits for the appending wave, the rest does not); new rows at
negative positions (length below q_len: skipped); a call split into several launches (q_len *
gqa > 16); and the 64K-context Q4_G64 step against the unfused step.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from block_quantized_kv_amd import (Layer, kvq_append, kvq_append_attend_decode, kvq_append_attend_decode_mq,
                                    kvq_attend_decode, kvq_attend_decode_mq)
from gpu_helpers import append_rows, rel_err

pytestmark = pytest.mark.gpu
TOL = 1e-3
SAME = 5e-4
CODECS = ["q8_0", "q4_0", "q4_g64"]


def _same_cache(a: Layer, b: Layer):
    for pa, pb, name in ((a.k, b.k, "K"), (a.v, b.v, "V")):
        assert torch.equal(pa.codes, pb.codes), f"{name} codes differ"
        assert torch.equal(pa.scales, pb.scales), f"{name} scales differ"


def _case(gpu, kc, vc, d, hq, hkv, lens, q_len=1, seed=0, max_len=None):
    rng = np.random.default_rng(seed)
    S = len(lens)
    cap = max(32, (max(lens) + 31) // 32 * 32)
    ml = max_len if max_len is not None else max(max(lens), 1)
    k = rng.standard_normal((S, cap, hkv, d)).astype(np.float32)
    v = rng.standard_normal((S, cap, hkv, d)).astype(np.float32)
    q = rng.standard_normal((S, q_len, hq, d)).astype(np.float32)
    # new rows: entry i of sequence s is position lens[s] - q_len + i; entries
    # at negative positions hold values that must never reach the cache
    kn = rng.standard_normal((S, q_len, hkv, d)).astype(np.float32)
    vn = rng.standard_normal((S, q_len, hkv, d)).astype(np.float32)
    for s, n in enumerate(lens):
        for i in range(q_len):
            p = n - q_len + i
            if p >= 0:
                kn[s, i], vn[s, i] = k[s, p], v[s, p]
    fused = Layer.create(kc, vc, d, hkv, S, cap, device=gpu)
    for s, n in enumerate(lens):
        old = max(n - q_len, 0)
        if old:
            append_rows(fused, torch.from_numpy(k[s, :old]).to(gpu), torch.from_numpy(v[s, :old]).to(gpu), s, 0)
    plain = fused.clone()
    torch.cuda.synchronize()

    # unfused reference: kvq_append of the new rows, then the attention
    sq, pos, rk, rv = [], [], [], []
    for s, n in enumerate(lens):
        for i in range(q_len):
            p = n - q_len + i
            if p >= 0:
                sq.append(s)
                pos.append(p)
                rk.append(kn[s, i])
                rv.append(vn[s, i])
    if sq:
        kvq_append(plain, torch.from_numpy(np.stack(rk)).to(gpu), torch.from_numpy(np.stack(rv)).to(gpu),
                   torch.tensor(sq, dtype=torch.int32, device=gpu), torch.tensor(pos, dtype=torch.int64, device=gpu))
    lens_t = torch.tensor(lens, dtype=torch.int64, device=gpu)
    scale = 1.0 / np.sqrt(d)
    qd = torch.from_numpy(q).to(gpu)
    kd, vd = torch.from_numpy(kn).to(gpu), torch.from_numpy(vn).to(gpu)
    if q_len == 1:
        ref_out = kvq_attend_decode(plain, qd[:, 0].contiguous(), lens_t, ml, scale).cpu().numpy()[:, None]
        out = kvq_append_attend_decode(fused, kd[:, 0].contiguous(), vd[:, 0].contiguous(), qd[:, 0].contiguous(),
                                       lens_t, ml, scale).cpu().numpy()[:, None]
    else:
        ref_out = kvq_attend_decode_mq(plain, qd, lens_t, ml, scale).cpu().numpy()
        out = kvq_append_attend_decode_mq(fused, kd, vd, qd, lens_t, ml, scale).cpu().numpy()
    _same_cache(fused, plain)
    assert np.isfinite(out).all()
    if np.abs(ref_out).max() > 0:
        assert rel_err(out, ref_out) <= SAME
    else:
        assert np.array_equal(out, ref_out)

    for s, n in enumerate(lens):
        kh = oracle.quant_dequant(kc, np.ascontiguousarray(k[s].transpose(1, 0, 2)))
        vh = oracle.quant_dequant(vc, np.ascontiguousarray(v[s].transpose(1, 0, 2)))
        for i in range(q_len):
            rows = min(n, ml) - q_len + i + 1
            if rows <= 0:
                assert np.array_equal(out[s, i], np.zeros_like(out[s, i])), (s, i)
                continue
            ref = oracle.attend_decode(q[s, i], kh, vh, rows, scale)
            err = rel_err(out[s, i], ref)
            assert err <= TOL, (kc, vc, d, hq, hkv, n, q_len, i, err)


@pytest.mark.parametrize("kc", CODECS)
@pytest.mark.parametrize("vc", CODECS)
def test_codec_pairs(gpu, kc, vc):
    d = {"q8_0": 64, "q4_0": 128, "q4_g64": 256}[kc]
    _case(gpu, kc, vc, d, hq=8, hkv=2, lens=[300, 33], seed=CODECS.index(kc) * 3 + CODECS.index(vc))


@pytest.mark.parametrize("q_len", [1, 3])
def test_f16_control_codec(gpu, q_len):
    # the f16 control codec through the fused append + decode
    _case(gpu, "f16", "f16", 128, hq=8, hkv=2, lens=[300, 33, 1], q_len=q_len, seed=16 + q_len)


@pytest.mark.parametrize("n", [1, 31, 32, 33, 255, 256, 257, 511, 513, 2000])
def test_new_row_positions(gpu, n):
    # small caches split every 256 rows: 256 ends a split, 257 opens one
    _case(gpu, "q4_g64", "q4_0", 128, hq=6, hkv=2, lens=[n], seed=n)


def test_mixed_lengths_with_an_empty_sequence(gpu):
    _case(gpu, "q8_0", "q4_g64", 128, hq=8, hkv=4, lens=[700, 0, 1, 257], seed=5)


@pytest.mark.parametrize("q_len,n", [(2, 257), (2, 33), (3, 33), (3, 258), (3, 2), (4, 1)])
def test_several_new_rows(gpu, q_len, n):
    # rows across a split (255 | 256) and a block (31 | 32) boundary, and rows
    # at negative positions when the sequence is shorter than q_len
    _case(gpu, "q4_0", "q8_0", 64, hq=4, hkv=1, lens=[n, 40], q_len=q_len, seed=q_len * 100 + n)


def test_several_launches(gpu):
    # gqa 8 with 3 queries: two launches; only the first one appends
    _case(gpu, "q4_g64", "q4_g64", 256, hq=16, hkv=2, lens=[600], q_len=3, seed=77)


def test_many_splits(gpu):
    _case(gpu, "q8_0", "q4_0", 128, hq=32, hkv=8, lens=[20000, 3001], seed=9)


@pytest.mark.parametrize("kc,vc,d", [("q8_0", "q4_0", 128), ("q4_g64", "q4_g64", 256), ("q4_0", "q4_g64", 64),
                                     ("q8_0", "q8_0", 128)])
def test_new_row_deep_in_a_long_split(gpu, kc, vc, d):
    # 8 kv-heads x 20668 rows give 768-row splits; the last one holds 700 rows
    # (22 blocks) with the new row in its last block, so the blocks that the
    # prologue streams never include it and, with a one-block ring, only the
    # blocks near the new row wait for the appending wave's stores
    _case(gpu, kc, vc, d, hq=16, hkv=8, lens=[26 * 768 + 700], seed=d + CODECS.index(kc))


def test_workload_64k_step_matches_unfused(gpu):
    """The 64K-context Q4_G64 decode step: one fused call against kvq_append +
    kvq_attend_decode on a copy of the same cache."""
    cfg = workloads.DECODE_64K
    n, H, d = cfg.ctx, cfg.n_kv_heads, cfg.head_dim
    kc, vc = cfg.layers[0]
    fused = Layer.create(kc, vc, d, H, 1, cfg.capacity, device=gpu)
    k = workloads.kv_rows(cfg, 0, 0, "k", 0, n, gpu)
    v = workloads.kv_rows(cfg, 0, 0, "v", 0, n, gpu)
    append_rows(fused, k[: n - 1], v[: n - 1], 0, 0)
    plain = fused.clone()
    q = workloads.queries(cfg, 0, gpu)
    lens = torch.tensor([n], dtype=torch.int64, device=gpu)
    kvq_append(plain, k[n - 1:].contiguous(), v[n - 1:].contiguous(), torch.zeros(1, dtype=torch.int32, device=gpu),
               torch.tensor([n - 1], dtype=torch.int64, device=gpu))
    ref = kvq_attend_decode(plain, q, lens, n, cfg.scale).cpu().numpy()
    out = kvq_append_attend_decode(fused, k[n - 1:].contiguous(), v[n - 1:].contiguous(), q, lens, n,
                                   cfg.scale).cpu().numpy()
    _same_cache(fused, plain)
    assert np.isfinite(out).all()
    assert rel_err(out, ref) <= SAME


def test_bounded_wait_that_runs_out_is_reported(gpu):
    """The fused append's wait for the appending wave is bounded: with the
    appending wave held from signalling (a test switch) and a 16-poll bound,
    the waves that read the new row's block give up, go on, and store
    KVQ_EWAIT; the kernel ends normally and the new row is still stored as
    kvq_append stores it."""
    from block_quantized_kv_amd import KVQ_EWAIT, kvq_debug_append_wait
    cfg = workloads.DECODE_64K  # 1024-row splits: the new row's block is read late in its split
    n, H, d = cfg.ctx, cfg.n_kv_heads, cfg.head_dim
    kc, vc = cfg.layers[0]
    L = Layer.create(kc, vc, d, H, 1, cfg.capacity, device=gpu)
    k = workloads.kv_rows(cfg, 0, 0, "k", 0, n, gpu)
    v = workloads.kv_rows(cfg, 0, 0, "v", 0, n, gpu)
    append_rows(L, k[: n - 1], v[: n - 1], 0, 0)
    q = workloads.queries(cfg, 0, gpu)
    lens = torch.tensor([n], dtype=torch.int64, device=gpu)
    st = torch.zeros(1, dtype=torch.int32, device=gpu)
    kvq_debug_append_wait(16, hold_flag=True)
    try:
        out = kvq_append_attend_decode(L, k[n - 1:].contiguous(), v[n - 1:].contiguous(), q, lens, n, cfg.scale,
                                       dev_status=st)
        torch.cuda.synchronize()
    finally:
        kvq_debug_append_wait(1 << 20, hold_flag=False)
    assert st.item() == KVQ_EWAIT
    assert out.shape == q.shape
    from block_quantized_kv_amd import layout
    for plane, rows in ((L.k, k), (L.v, v)):
        codes, scales = layout.plane_to_rows(plane, seq=0)
        want_c, want_s = oracle.quantize_rows(plane.codec, rows[n - 1].cpu().numpy())
        assert np.array_equal(codes[0, :, n - 1], want_c) and np.array_equal(scales[0, :, n - 1], want_s)
    # with the default bound the same call stores nothing
    st.zero_()
    kvq_append_attend_decode(L, k[n - 1:].contiguous(), v[n - 1:].contiguous(), q, lens, n, cfg.scale,
                             dev_status=st)
    torch.cuda.synchronize()
    assert st.item() == 0
