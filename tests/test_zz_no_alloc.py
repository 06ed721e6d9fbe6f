"""The no-allocation decode entry point, kvq_append_attend_decode_noalloc:
its split partials live in the library's own device scratch instead of a
caller workspace.  Checked through the C ABI against kvq_append_attend_decode
(the same call with a workspace) on a copy of the same cache: the cache bytes
equal, the outputs within 5e-4 of max|out| (the waves of a split take blocks
in arrival order, so the two runs may round differently), and both within
the decode bar, 1e-3 of max|oracle|.  Two calls in a row, the second with a
smaller input (fewer sequences, a shorter context, other head counts), so
the scratch's contents from the first call must not leak into the second."""
import numpy as np
import pytest
import torch

import oracle
from block_quantized_kv_amd import (Layer, kvq_append_attend_decode, kvq_append_attend_decode_noalloc,
                                    kvq_noalloc_scratch_bytes)
from gpu_helpers import append_rows, oracle_decode_all, rel_err

pytestmark = pytest.mark.gpu
TOL = 1e-3
SAME = 5e-4


def _call(gpu, kc, vc, d, hq, hkv, lens, seed):
    rng = np.random.default_rng(seed)
    S = len(lens)
    cap = max(32, (max(lens) + 31) // 32 * 32)
    k = rng.standard_normal((S, cap, hkv, d)).astype(np.float32)
    v = rng.standard_normal((S, cap, hkv, d)).astype(np.float32)
    q = rng.standard_normal((S, hq, d)).astype(np.float32)
    with_ws = Layer.create(kc, vc, d, hkv, S, cap, device=gpu)
    for s, n in enumerate(lens):
        if n > 1:
            append_rows(with_ws, torch.from_numpy(k[s, :n - 1]).to(gpu), torch.from_numpy(v[s, :n - 1]).to(gpu), s, 0)
    no_ws = with_ws.clone()
    kn = torch.from_numpy(np.stack([k[s, max(n - 1, 0)] for s, n in enumerate(lens)])).to(gpu)
    vn = torch.from_numpy(np.stack([v[s, max(n - 1, 0)] for s, n in enumerate(lens)])).to(gpu)
    qd = torch.from_numpy(q).to(gpu)
    lens_t = torch.tensor(lens, dtype=torch.int64, device=gpu)
    scale = 1.0 / np.sqrt(d)
    ref = kvq_append_attend_decode(with_ws, kn, vn, qd, lens_t, max(lens), scale)
    out = torch.full_like(qd, float("nan"))
    kvq_append_attend_decode_noalloc(no_ws, kn, vn, qd, lens_t, max(lens), scale, out)
    torch.cuda.synchronize()
    for pa, pb in ((no_ws.k, with_ws.k), (no_ws.v, with_ws.v)):
        assert torch.equal(pa.codes, pb.codes) and torch.equal(pa.scales, pb.scales)
    got, want = out.cpu().numpy(), ref.cpu().numpy()
    assert np.isfinite(got).all()
    assert rel_err(got, want) <= SAME
    for s, n in enumerate(lens):
        r = oracle_decode_all(kc, vc, q[s], k[s], v[s], n, scale)
        assert rel_err(got[s], r) <= TOL, (s, n)


def test_noalloc_matches_workspace_call_twice(gpu):
    # first call: 3 sequences up to 20000 rows (many splits per kv-head)
    _call(gpu, "q4_g64", "q4_g64", 256, 24, 4, [20000, 7001, 1], seed=1)
    # second call, smaller: one sequence of 700 rows, other codecs and heads
    _call(gpu, "q8_0", "q4_0", 128, 8, 2, [700], seed=2)


def test_noalloc_rejects_calls_beyond_its_scratch(gpu):
    from block_quantized_kv_amd import KvqError, kvq_decode_workspace_bytes
    L = Layer.create("q8_0", "q4_0", 128, 8, 64, 131072, device=gpu)
    need = kvq_decode_workspace_bytes(L, 32, 64, 131072)
    assert need > kvq_noalloc_scratch_bytes()
    q = torch.zeros(64, 32, 128, device=gpu)
    kv = torch.zeros(64, 8, 128, device=gpu)
    with pytest.raises(KvqError) as e:
        kvq_append_attend_decode_noalloc(L, kv, kv, q, torch.full((64,), 131072, device=gpu), 131072, 0.1,
                                         torch.empty_like(q))
    assert e.value.status == 4
