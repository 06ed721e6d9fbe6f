"""Calls from several host threads at once, each thread with its own stream,
cache, workspace and status word.  The library keeps no per-call state
outside its arguments, and ctypes releases the GIL during a call, so the
threads' launches really interleave: every thread's outputs must equal the
same calls run one thread at a time (to the rounding the dynamic block
hand-out inside a split allows, 5e-4) and the oracle's (1e-3), and no status
word may be set."""
import threading

import numpy as np
import pytest
import torch

import oracle
from block_quantized_kv_amd import Layer, decode_workspace, kvq_append, kvq_append_attend_decode
from gpu_helpers import rel_err

pytestmark = pytest.mark.gpu
STEPS = 24
CASES = [  # (k codec, v codec, head_dim, kv-heads, q-heads, prefix rows)
    ("q4_g64", "q4_g64", 256, 4, 24, 8000),
    ("q8_0", "q4_0", 128, 8, 32, 5000),
    ("q8_0", "q4_g64", 64, 1, 4, 300),
]


def _case(gpu, idx):
    kc, vc, d, hkv, hq, n = CASES[idx]
    rng = np.random.default_rng(100 + idx)
    rows = n + STEPS
    k = rng.standard_normal((rows, hkv, d)).astype(np.float32)
    v = rng.standard_normal((rows, hkv, d)).astype(np.float32)
    q = rng.standard_normal((STEPS, 1, hq, d)).astype(np.float32)
    layer = Layer.create(kc, vc, d, hkv, 1, (rows + 31) // 32 * 32, device=gpu)
    kvq_append(layer, torch.from_numpy(k[:n]).to(gpu), torch.from_numpy(v[:n]).to(gpu),
               torch.zeros(n, dtype=torch.int32, device=gpu), torch.arange(n, dtype=torch.int64, device=gpu))
    torch.cuda.synchronize()
    dev = dict(k_new=torch.from_numpy(k[n:]).to(gpu).unsqueeze(1), v_new=torch.from_numpy(v[n:]).to(gpu).unsqueeze(1),
               q=torch.from_numpy(q).to(gpu),
               lens=[torch.tensor([n + i + 1], dtype=torch.int64, device=gpu) for i in range(STEPS)])
    torch.cuda.synchronize()
    return dict(kc=kc, vc=vc, d=d, hq=hq, n=n, k=k, v=v, q=q, layer=layer, dev=dev)


def _steps(gpu, c, stream):
    """The case's STEPS fused append + decode steps on `stream`: outputs and
    the status word."""
    n, hq, d = c["n"], c["hq"], c["d"]
    with torch.cuda.stream(stream):
        ws = decode_workspace(c["layer"], hq, 1, n + STEPS)
        status = torch.zeros(1, dtype=torch.int32, device=gpu)
        outs = torch.empty(STEPS, 1, hq, d, device=gpu)
        for i in range(STEPS):
            kvq_append_attend_decode(c["layer"], c["dev"]["k_new"][i], c["dev"]["v_new"][i], c["dev"]["q"][i],
                                     c["dev"]["lens"][i], n + i + 1, 1.0 / np.sqrt(d), out=outs[i], workspace=ws,
                                     dev_status=status)
        stream.synchronize()
    return outs.cpu().numpy(), int(status.item())


def test_concurrent_calls_from_threads(gpu):
    cases = [_case(gpu, i) for i in range(len(CASES))]
    streams = [torch.cuda.Stream(device=gpu) for _ in cases]
    results, errors = [None] * len(cases), []

    def worker(i):
        try:
            results[i] = _steps(gpu, cases[i], streams[i])
        except Exception as e:  # reported below, in the test's own thread
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    # the same steps, one case at a time (they rewrite the same rows with the
    # same values, so the cache is unchanged)
    alone = [_steps(gpu, c, torch.cuda.current_stream(gpu)) for c in cases]
    for i, c in enumerate(cases):
        out, status = results[i]
        ref_out, ref_status = alone[i]
        assert status == 0 and ref_status == 0, (i, status, ref_status)
        assert rel_err(out, ref_out) <= 5e-4, i
        kh = oracle.quant_dequant(c["kc"], np.ascontiguousarray(c["k"].transpose(1, 0, 2)))
        vh = oracle.quant_dequant(c["vc"], np.ascontiguousarray(c["v"].transpose(1, 0, 2)))
        for s in (0, STEPS // 2, STEPS - 1):
            ref = oracle.attend_decode(c["q"][s, 0], kh, vh, c["n"] + s + 1, 1.0 / np.sqrt(c["d"]))
            assert rel_err(out[s, 0], ref) <= 1e-3, (i, s)
