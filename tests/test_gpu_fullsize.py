"""Full-size decode parity: every output of the workload configurations,
compared directly with the oracle (binary64 attention over the oracle's own
quantization of the same fp32 rows), at the decode bar max|gpu - oracle| /
max|oracle| <= 1e-3 over the outputs of one call (per layer for the
four-layer 196K configuration).

  * the timed 64K-context step itself: the cache built exactly as the
    benchmark builds it (its own setup function), then one
    kvq_append_attend_decode call appending row 65535 and attending over
    65536 rows, eager and as HIP-graph replays; all 24 q-heads, and the
    appended row's codes and scales bit for bit;
  * the 32K context, q8_0 K / q4_0 V with outlier channels: all 32 q-heads;
  * the 196K context, four layers (q8_0 / q8_0, then three Q4_G64 / Q4_G64):
    all 24 q-heads of every layer;
  * 16 sequences of 4K..128K rows, q8_0 K / q4_0 V: all 32 q-heads of every
    sequence;
  * the 64K context with two drafted tokens per step: all 24 q-heads of both
    queries.
Each test prints its measured error.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from block_quantized_kv_amd import Layer, kvq_append_attend_decode_mq, kvq_attend_decode, kvq_attend_decode_mq, layout
from gpu_helpers import append_rows, oracle_decode_all, pool, rel_err, report

pytestmark = pytest.mark.gpu
TOL = 1e-3


def test_timed_64k_step_all_heads(gpu, capsys):
    import bench
    hs = bench.headline_setup(torch, gpu, rotate=1, keep_host=True)
    cfg = hs.cfg
    kc, vc = cfg.layers[0]
    n, H = cfg.ctx, cfg.n_kv_heads
    k_host, v_host = hs.host_kv
    ref = oracle_decode_all(kc, vc, hs.q[0].cpu().numpy(), k_host, v_host, n, cfg.scale)

    # eager: one call
    hs.step(0)
    torch.cuda.synchronize()
    eager = hs.out.cpu().numpy()[0]
    assert np.isfinite(eager).all()
    err = rel_err(eager, ref)
    report(capsys, "64K step, kvq_append_attend_decode eager, 24 q-heads", err, TOL)
    assert err <= TOL

    # the appended row (65535) equals the oracle's quantization, every kv-head
    for plane, rows in ((hs.base.k, k_host), (hs.base.v, v_host)):
        codes, scales = layout.plane_to_rows(plane, seq=0)
        want_c, want_s = oracle.quantize_rows(plane.codec, rows[n - 1])
        assert np.array_equal(codes[0, :, n - 1], want_c)
        assert np.array_equal(scales[0, :, n - 1], want_s)

    # as the benchmark replays it: a captured step, replayed several times
    # with eager work in between; every replay against the oracle
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            hs.step(0, cap)
    torch.cuda.synchronize()
    worst = 0.0
    for i in range(3):
        hs.out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = hs.out.cpu().numpy()[0]
        assert np.isfinite(got).all()
        worst = max(worst, rel_err(got, ref))
        hs.step(0)  # eager work between replays
        torch.cuda.synchronize()
    report(capsys, "64K step, HIP-graph replays, 24 q-heads", worst, TOL)
    assert worst <= TOL


def _all_heads(gpu, capsys, cfg, layer_idx=0):
    """Every (sequence, q-head) output of one layer of cfg against the oracle."""
    kc, vc = cfg.layers[layer_idx]
    lens = workloads.seq_lengths(cfg, "cpu").tolist()
    layer = Layer.create(kc, vc, cfg.head_dim, cfg.n_kv_heads, cfg.n_seqs, cfg.capacity, device=gpu)
    for s, n in enumerate(lens):
        k = workloads.kv_rows(cfg, layer_idx, s, "k", 0, n, gpu)
        v = workloads.kv_rows(cfg, layer_idx, s, "v", 0, n, gpu)
        append_rows(layer, k, v, s, 0)
        del k, v
    q = workloads.queries(cfg, layer_idx, gpu)
    out = kvq_attend_decode(layer, q, torch.tensor(lens, dtype=torch.int64, device=gpu), max(lens),
                            cfg.scale).cpu().numpy()
    del layer
    qn = q.cpu().numpy()
    assert np.isfinite(out).all()
    refs = []
    for s, n in enumerate(lens):  # one sequence's rows on the host at a time
        k = workloads.kv_rows(cfg, layer_idx, s, "k", 0, n, gpu).cpu().numpy()
        v = workloads.kv_rows(cfg, layer_idx, s, "v", 0, n, gpu).cpu().numpy()
        refs.append(oracle_decode_all(kc, vc, qn[s], k, v, n, cfg.scale))
    err = rel_err(out, np.stack(refs))
    report(capsys, f"{cfg.name} layer {layer_idx} ({kc}/{vc}), {cfg.n_seqs} seq x {cfg.n_q_heads} q-heads", err,
           TOL)
    assert err <= TOL, (cfg.name, layer_idx, err)


def test_decode_32k_all_heads(gpu, capsys):
    _all_heads(gpu, capsys, workloads.DECODE_32K)


@pytest.mark.parametrize("layer_idx", [0, 1, 2, 3])
def test_decode_196k_every_layer_all_heads(gpu, capsys, layer_idx):
    _all_heads(gpu, capsys, workloads.DECODE_196K, layer_idx)


def test_batched_16_sequences_all_heads(gpu, capsys):
    _all_heads(gpu, capsys, workloads.BATCHED)


def test_64k_two_queries_all_heads(gpu, capsys):
    """The 64K-context Q4_G64 decode with two drafted tokens per step
    (kvq_append_attend_decode_mq appends rows 65534 and 65535, then both
    queries attend): all 24 q-heads of both queries."""
    cfg = workloads.DECODE_64K
    n, H, d, hq = cfg.ctx, cfg.n_kv_heads, cfg.head_dim, cfg.n_q_heads
    kc, vc = cfg.layers[0]
    layer = Layer.create(kc, vc, d, H, 1, cfg.capacity, device=gpu)
    k = workloads.kv_rows(cfg, 0, 0, "k", 0, n, gpu)
    v = workloads.kv_rows(cfg, 0, 0, "v", 0, n, gpu)
    append_rows(layer, k[: n - 2], v[: n - 2], 0, 0)
    g = torch.Generator(device="cpu").manual_seed(77)
    q = torch.randn(1, 2, hq, d, generator=g).to(gpu)
    lens = torch.tensor([n], dtype=torch.int64, device=gpu)
    out = kvq_append_attend_decode_mq(layer, k[n - 2:].contiguous()[None], v[n - 2:].contiguous()[None], q, lens, n,
                                      cfg.scale).cpu().numpy()
    again = kvq_attend_decode_mq(layer, q, lens, n, cfg.scale).cpu().numpy()
    kn, vn, qn = k.cpu().numpy(), v.cpu().numpy(), q.cpu().numpy()
    worst = 0.0
    for i in range(2):
        ref = oracle_decode_all(kc, vc, qn[0, i], kn, vn, n - 1 + i, cfg.scale)
        worst = max(worst, rel_err(out[0, i], ref), rel_err(again[0, i], ref))
    report(capsys, "64K, two queries (fused append + attend, then attend), 24 q-heads each", worst, TOL)
    assert worst <= TOL
