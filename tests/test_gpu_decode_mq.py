"""GPU multi-query decode parity (several drafted tokens verified per step)
against the oracle: query i of a sequence with length L attends rows
[0, L - q_len + i], i.e. binary64 decode attention over the oracle's own
quantization with length L - q_len + i + 1 (zero rows -> output 0).

Bar: max|gpu - oracle| / max|oracle| <= 1e-3 per call, as for decode.
Covered: q_len 1-4 on every head_dim, GQA ratios whose q_len * gqa exceeds
one 16-column tile (several launches per call), the largest q_len (64), sequences shorter than
q_len, the newest rows alone in the last split, many splits, q_len = 1
against kvq_attend_decode bit for bit (the 64K Q4_G64 workload with two
queries per step, every head, is in test_gpu_fullsize.py).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from block_quantized_kv_amd import Layer, kvq_attend_decode, kvq_attend_decode_mq
from gpu_helpers import append_rows, rel_err

pytestmark = pytest.mark.gpu
TOL = 1e-3


def _case(gpu, kc, vc, d, hq, hkv, lens, q_len, seed=0, cap=None, max_len=None):
    rng = np.random.default_rng(seed)
    S = len(lens)
    cap = cap or max(32, (max(lens) + 31) // 32 * 32)
    layer = Layer.create(kc, vc, d, hkv, S, cap, device=gpu)
    q = rng.standard_normal((S, q_len, hq, d)).astype(np.float32)
    ks, vs = [], []
    for s, n in enumerate(lens):
        k = rng.standard_normal((cap, hkv, d)).astype(np.float32)
        v = rng.standard_normal((cap, hkv, d)).astype(np.float32)
        append_rows(layer, torch.from_numpy(k).to(gpu), torch.from_numpy(v).to(gpu), s, 0)
        ks.append(k)
        vs.append(v)
    scale = 1.0 / np.sqrt(d)
    ml = max_len if max_len is not None else max(lens)
    out = kvq_attend_decode_mq(layer, torch.from_numpy(q).to(gpu),
                               torch.tensor(lens, dtype=torch.int64, device=gpu), ml, scale).cpu().numpy()
    for s, n in enumerate(lens):
        kh = oracle.quant_dequant(kc, np.ascontiguousarray(ks[s].transpose(1, 0, 2)))
        vh = oracle.quant_dequant(vc, np.ascontiguousarray(vs[s].transpose(1, 0, 2)))
        for i in range(q_len):
            rows = n - q_len + i + 1
            if rows <= 0:
                assert np.array_equal(out[s, i], np.zeros_like(out[s, i])), (s, i)
                continue
            ref = oracle.attend_decode(q[s, i], kh, vh, rows, scale)
            err = rel_err(out[s, i], ref)
            assert np.isfinite(out[s, i]).all()
            assert err <= TOL, (kc, vc, d, hq, hkv, n, q_len, i, err)
    return layer, q, out


@pytest.mark.parametrize("q_len", [1, 2, 3, 4])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_query_counts_and_head_dims(gpu, q_len, d):
    _case(gpu, "q4_g64", "q8_0", d, hq=8, hkv=2, lens=[700, 37], q_len=q_len, seed=q_len * 7 + d)


@pytest.mark.parametrize("kc,vc", [("q8_0", "q4_0"), ("q4_0", "q4_g64"), ("q4_g64", "q4_g64"), ("q8_0", "q8_0")])
def test_codec_pairs_two_queries(gpu, kc, vc):
    _case(gpu, kc, vc, 128, hq=12, hkv=2, lens=[513, 64], q_len=2, seed=len(kc) * 10 + len(vc))


@pytest.mark.parametrize("gqa,q_len", [(6, 3), (8, 3), (16, 2), (5, 4), (1, 16), (2, 20)])
def test_more_columns_than_one_tile(gpu, gqa, q_len):
    # gqa * q_len > 16: the call runs several launches over the same K/V
    _case(gpu, "q8_0", "q4_0", 64, hq=2 * gqa, hkv=2, lens=[300], q_len=q_len, seed=gqa * 31 + q_len)


@pytest.mark.parametrize("gqa", [1, 4])
def test_the_largest_query_count(gpu, gqa):
    # q_len at the limit (KVQ_MAX_QUERIES = 64): 4 or 16 launches of 16
    # columns over the same K/V, the first queries of the shorter sequence
    # seeing nothing
    _case(gpu, "q8_0", "q4_g64", 128, hq=2 * gqa, hkv=2, lens=[900, 40], q_len=64, seed=64 + gqa)


def test_sequences_shorter_than_the_queries(gpu):
    # length 1 and 2 with 4 queries: the first queries see nothing (output 0)
    _case(gpu, "q4_0", "q4_0", 128, hq=4, hkv=1, lens=[1, 2, 4, 5], q_len=4, seed=11)


def test_newest_rows_alone_in_the_last_split(gpu):
    # 8193 rows over 256-row splits (max_len 16384 forces 8-block splits ...):
    # the last split holds a single row, visible to the last query only
    _case(gpu, "q4_g64", "q4_g64", 128, hq=8, hkv=2, lens=[8193, 8194], q_len=3, seed=5, cap=16384,
          max_len=16384)


def test_many_splits(gpu):
    _case(gpu, "q8_0", "q4_0", 128, hq=32, hkv=8, lens=[20000, 3000], q_len=2, seed=9)


def test_one_query_matches_plain_decode_bitwise(gpu):
    layer, q, out = _case(gpu, "q4_g64", "q4_0", 256, hq=12, hkv=2, lens=[2000, 100], q_len=1, seed=3)
    q1 = torch.from_numpy(q[:, 0]).to(gpu)
    lens = torch.tensor([2000, 100], dtype=torch.int64, device=gpu)
    plain = kvq_attend_decode(layer, q1, lens, 2000, 1.0 / 16.0).cpu().numpy()
    assert np.array_equal(plain, out[:, 0])
