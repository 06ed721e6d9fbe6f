"""GPU chunked-prefill parity against the oracle (binary64 causal attention over
the oracle's own quantization of the same rows; bf16 queries widened exactly).

Bar: max|gpu - oracle| / max|oracle| <= 1e-2, the prefill tolerance (the
matrix cores see K_hat, V_hat, the scaled query and P rounded to binary16).
Covered: the tiny prefill enumerated in full, ragged prefix/chunk lengths,
every codec pair, head_dim 64/128/256, several GQA ratios, a chunk at
position 0, queries far outside the binary16 range, negative and zero softmax scales, the chunk of a middle sequence of a three-sequence
cache over several workgroups at every head_dim, the 64K model's heads at head_dim 256 (ragged column groups,
and the 2048-token chunk over 32768 rows sampled at every column-group boundary), graph replays against the
eager call, and the 2048-token chunk over a 32768-token prefix on every one of its 65536 (token, head) rows.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from block_quantized_kv_amd import Layer, kvq_attend_prefill
from gpu_helpers import append_rows, pool, rel_err, report

pytestmark = pytest.mark.gpu
TOL = 1e-2
CODECS = ["q8_0", "q4_0", "q4_g64"]


def _run(gpu, kc, vc, d, hq, hkv, P, T, seed=0, sample=None, cap_extra=0, qmul=1.0, capsys=None, scale_mul=1.0):
    q, k, v = workloads.prefill_inputs(gpu, seed_layer=seed, prefix=P, chunk=T, n_q_heads=hq,
                                       n_kv_heads=hkv, head_dim=d)
    if qmul != 1.0:  # a power of two: exact in bf16
        q = (q.float() * qmul).to(torch.bfloat16)
    cap = (P + T + 31) // 32 * 32 + cap_extra
    layer = Layer.create(kc, vc, d, hkv, 1, cap, device=gpu)
    append_rows(layer, k, v, 0, 0)                      # prefix and chunk rows
    scale = 1.0 / np.sqrt(d) / qmul * scale_mul
    out = kvq_attend_prefill(layer, q, 0, P, scale).cpu().numpy()
    kh = oracle.quant_dequant(kc, k.cpu().numpy().transpose(1, 0, 2).copy())
    vh = oracle.quant_dequant(vc, v.cpu().numpy().transpose(1, 0, 2).copy())
    qn = q.float().cpu().numpy()
    if sample is None:
        ref = oracle.attend_prefill(qn, kh, vh, P, scale)
        got = out
    else:
        toks, heads = sample
        # the sample in pieces, side by side on the host's cores
        pieces = np.array_split(np.arange(len(toks)), 64)
        parts = pool().map(lambda ix: oracle.attend_prefill(qn, kh, vh, P, scale, tokens=toks[ix], heads=heads[ix]),
                           pieces)
        ref = np.concatenate(list(parts))
        got = out[toks, heads]
    err = rel_err(got, ref)
    if capsys is not None:
        report(capsys, f"prefill {T} tokens over a {P}-row prefix ({kc}/{vc}, d {d}, {hq}/{hkv} heads), "
                       f"{len(got) if sample is not None else T * hq} (token, head) rows", err, TOL)
    assert np.isfinite(out).all()
    assert err <= TOL, (kc, vc, d, hq, hkv, P, T, err)
    return err


def test_tiny_prefill_enumerated(gpu):
    _run(gpu, "q8_0", "q4_0", 128, 32, 8, 64, 16)


@pytest.mark.parametrize("kc", CODECS)
@pytest.mark.parametrize("vc", CODECS)
def test_codec_pairs(gpu, kc, vc):
    d = {"q8_0": 64, "q4_0": 128, "q4_g64": 256}[vc]
    _run(gpu, kc, vc, d, 8, 2, 100, 37, seed=CODECS.index(kc) * 3 + CODECS.index(vc))


@pytest.mark.parametrize("P,T", [(0, 1), (0, 70), (1, 1), (31, 33), (63, 65), (200, 300), (1000, 129)])
def test_ragged_lengths(gpu, P, T):
    _run(gpu, "q4_g64", "q8_0", 128, 6, 1, P, T, seed=P + T)


@pytest.mark.parametrize("gqa", [1, 3, 4, 16])
def test_gqa_ratios(gpu, gqa):
    _run(gpu, "q8_0", "q4_0", 64, 2 * gqa, 2, 90, 50, seed=gqa)


@pytest.mark.parametrize("qmul", [2.0 ** -30, 2.0 ** 40])
def test_query_outside_binary16_range(gpu, qmul):
    # bf16 queries far below and above the binary16 range: each (token, head)
    # column is scaled by a power of two before the binary16 rounding, and the
    # softmax scale divided by qmul makes the exact result the unscaled one
    _run(gpu, "q8_0", "q4_g64", 128, 8, 2, 70, 45, seed=11, qmul=qmul)


@pytest.mark.parametrize("scale_mul", [-1.0, 0.0, -0.0, 3.0])
def test_softmax_scale_sign_and_zero(gpu, scale_mul):
    # any non-NaN scale: a negative one favours the smallest scores, a zero
    # one weighs every visible row alike (the mean of V_hat up to the diagonal)
    _run(gpu, "q8_0", "q4_0", 128, 8, 2, 70, 45, seed=13, scale_mul=scale_mul)


def test_xcd_placement_of_column_groups(gpu):
    # 8 kv-heads x 3 column groups of 256 (token, head) columns: 24 workgroups,
    # dealt to the XCDs by a permutation that keeps each kv-head's groups
    # together; every (kv-head, column group) pair must still be computed once
    _run(gpu, "q8_0", "q4_0", 128, 16, 8, 500, 300, seed=17)


def test_capacity_slack_rows_ignored(gpu):
    # capacity beyond the chunk: never-written rows after it must not matter
    _run(gpu, "q8_0", "q4_0", 128, 8, 2, 40, 30, cap_extra=64)


def test_workload_prefill_2048_over_32768(gpu, capsys):
    """The chunked-prefill workload (q8_0 K / q4_0 V, 32/8 heads, d 128), in
    the launch configuration the benchmark times, against the oracle on every
    one of its 65536 (token, head) rows (the oracle's rows run side by side on
    the host's cores)."""
    W = workloads.PREFILL
    P, T, hq = W["prefix"], W["chunk"], W["n_q_heads"]
    toks = np.repeat(np.arange(T), hq)
    heads = np.tile(np.arange(hq), T)
    _run(gpu, W["k_codec"], W["v_codec"], W["head_dim"], hq, W["n_kv_heads"], P, T, sample=(toks, heads),
         capsys=capsys)


@pytest.mark.parametrize("kc,vc", [("q4_g64", "q4_g64"), ("q8_0", "q4_0")])
def test_head_dim_256_model_heads(gpu, kc, vc):
    # the 64K model's heads (24/4, d 256) run 12-wave workgroups of 192
    # (token, head) columns: 300 tokens x 6 heads = 1800 columns per kv-head
    # make 10 column groups (the last one ragged), 40 workgroups dealt to the
    # XCDs by kv-head
    _run(gpu, kc, vc, 256, 24, 4, 500, 300, seed=21 + len(kc))


def test_head_dim_256_chunk_2048_over_32768_sampled(gpu, capsys):
    """The 2048-token chunk over a 32768-row prefix with the 64K model's heads
    (24/4, d 256, Q4_G64): 256 workgroups of 192 columns, one per compute
    unit.  Checked against the oracle on every column on either side of each
    192-column group boundary of kv-heads 0 and 3, and on 64 evenly spaced
    tokens with all 24 heads."""
    P, T, hq, hkv = 32768, 2048, 24, 4
    G = hq // hkv
    cols = []
    for kvh in (0, hkv - 1):
        for i in range(1, T * G // 192):
            cols += [(kvh, 192 * i - 1), (kvh, 192 * i)]
    toks = [c // G for _, c in cols]
    heads = [kvh * G + c % G for kvh, c in cols]
    for t in np.linspace(0, T - 1, 64).astype(int):
        toks += [int(t)] * hq
        heads += list(range(hq))
    _run(gpu, "q4_g64", "q4_g64", 256, hq, hkv, P, T, seed=23, sample=(np.array(toks), np.array(heads)),
         capsys=capsys)


@pytest.mark.parametrize("kc,vc,d", [("q4_0", "q8_0", 64), ("q8_0", "q4_0", 128), ("q4_g64", "q4_g64", 256)])
def test_middle_sequence_over_several_workgroups(gpu, kc, vc, d):
    # the chunk of sequence 1 of a three-sequence cache whose neighbours hold
    # other rows (reading the wrong sequence shows), 4 x 200 (token, head)
    # columns per kv-head: several workgroups of columns, at every head_dim
    hq, hkv, P, T = 8, 2, 150, 200
    q, k, v = workloads.prefill_inputs(gpu, seed_layer=d, prefix=P, chunk=T, n_q_heads=hq, n_kv_heads=hkv,
                                       head_dim=d)
    cap = (P + T + 31) // 32 * 32
    layer = Layer.create(kc, vc, d, hkv, 3, cap, device=gpu)
    for s in (0, 2):
        _, ko, vo = workloads.prefill_inputs(gpu, seed_layer=d + 1 + s, prefix=P, chunk=T, n_q_heads=hq,
                                             n_kv_heads=hkv, head_dim=d)
        append_rows(layer, 4.0 * ko, -3.0 * vo, s, 0)
    append_rows(layer, k, v, 1, 0)
    scale = 1.0 / np.sqrt(d)
    out = kvq_attend_prefill(layer, q, 1, P, scale).cpu().numpy()
    kh = oracle.quant_dequant(kc, k.cpu().numpy().transpose(1, 0, 2).copy())
    vh = oracle.quant_dequant(vc, v.cpu().numpy().transpose(1, 0, 2).copy())
    ref = oracle.attend_prefill(q.float().cpu().numpy(), kh, vh, P, scale)
    assert np.isfinite(out).all()
    err = rel_err(out, ref)
    assert err <= TOL, (kc, vc, d, err)


def test_graph_replay_matches_eager(gpu):
    """kvq_attend_prefill captured in a HIP graph: every replay equals the
    eager call bit for bit (the call only enqueues its kernel), with eager
    work on the device between the replays."""
    d, hq, hkv, P, T = 128, 8, 2, 300, 130
    q, k, v = workloads.prefill_inputs(gpu, seed_layer=23, prefix=P, chunk=T, n_q_heads=hq, n_kv_heads=hkv,
                                       head_dim=d)
    layer = Layer.create("q8_0", "q4_0", d, hkv, 1, (P + T + 31) // 32 * 32, device=gpu)
    append_rows(layer, k, v, 0, 0)
    out = torch.empty(T, hq, d, device=gpu)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        kvq_attend_prefill(layer, q, 0, P, d ** -0.5, out=out)
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        kvq_attend_prefill(layer, q, 0, P, d ** -0.5, out=out)
    for i in range(4):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), i
        kvq_attend_prefill(layer, q, 0, P, 0.5 * d ** -0.5)  # eager work between replays
