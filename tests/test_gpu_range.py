"""The binary16 operand range of the attention calls.

Decode rounds each dequantized V value to binary16, prefill each K and V
value, so |x_hat| must stay within 65504.  A group whose scale could break
that (4-bit: dq >= 8192, q8_0: dq >= 512; values from about 57000 / 65000)
is reported through the call's device status word as KVQ_EOVERFLOW; below
it the call matches the oracle and stores nothing.  Decode's K enters with
its scale applied in fp32, so large keys stay exact.  Every kernel here
exits normally: the status is a store, not a trap.
"""
import numpy as np
import pytest
import torch

import oracle
from block_quantized_kv_amd import (KVQ_EOVERFLOW, Layer, kvq_append, kvq_append_attend_decode, kvq_attend_decode,
                                    kvq_attend_prefill)
from gpu_helpers import append_rows, rel_err

pytestmark = pytest.mark.gpu


def _layer(gpu, kc, vc, d, H, n, k, v):
    cap = (n + 31) // 32 * 32
    L = Layer.create(kc, vc, d, H, 1, cap, device=gpu)
    append_rows(L, torch.from_numpy(k).to(gpu), torch.from_numpy(v).to(gpu), 0, 0)
    return L


def _decode(gpu, kc, vc, kmul, vmul, seed):
    rng = np.random.default_rng(seed)
    d, H, hq, n = 128, 2, 8, 700
    k = rng.standard_normal((n, H, d)).astype(np.float32)
    v = rng.standard_normal((n, H, d)).astype(np.float32)
    # a run of rows (whole groups) at the tested magnitude, |x| <= 4.5 x mul
    k[100:140] = np.clip(k[100:140], -4.5, 4.5) * kmul
    v[300:340] = np.clip(v[300:340], -4.5, 4.5) * vmul
    L = _layer(gpu, kc, vc, d, H, n, k, v)
    q = rng.standard_normal((1, hq, d)).astype(np.float32)
    st = torch.zeros(1, dtype=torch.int32, device=gpu)
    out = kvq_attend_decode(L, torch.from_numpy(q).to(gpu), torch.tensor([n], device=gpu), n, 1 / np.sqrt(d),
                            dev_status=st).cpu().numpy()
    kh = oracle.quant_dequant(kc, np.ascontiguousarray(k.transpose(1, 0, 2)))
    vh = oracle.quant_dequant(vc, np.ascontiguousarray(v.transpose(1, 0, 2)))
    ref = oracle.attend_decode(q[0], kh, vh, n, 1 / np.sqrt(d))
    return int(st.item()), out[0], ref


@pytest.mark.parametrize("vc,vmul", [("q4_g64", 12000.0), ("q4_0", 12000.0), ("q8_0", 14000.0)])
def test_decode_values_inside_the_range_match(gpu, vc, vmul):
    # |v| up to ~4.5 sigma x vmul stays below the reporting threshold
    status, out, ref = _decode(gpu, "q8_0", vc, 1.0, vmul, seed=1)
    assert status == 0
    assert np.isfinite(out).all() and rel_err(out, ref) <= 1e-3


@pytest.mark.parametrize("vc", ["q4_g64", "q4_0", "q8_0"])
def test_decode_values_beyond_the_range_are_reported(gpu, vc):
    status, out, _ = _decode(gpu, "q8_0", vc, 1.0, 1e5, seed=2)
    assert status == KVQ_EOVERFLOW


@pytest.mark.parametrize("kc", ["q4_g64", "q8_0"])
def test_decode_large_keys_stay_exact(gpu, kc):
    # K is scaled in fp32 after the matrix product: no range limit, no report
    status, out, ref = _decode(gpu, kc, "q4_0", 1e5, 1.0, seed=3)
    assert status == 0
    assert np.isfinite(out).all() and rel_err(out, ref) <= 1e-3


def test_fused_append_reports_a_new_row_beyond_the_range(gpu):
    rng = np.random.default_rng(4)
    d, H, hq, n = 128, 2, 8, 333
    k = rng.standard_normal((n, H, d)).astype(np.float32)
    v = rng.standard_normal((n, H, d)).astype(np.float32)
    L = _layer(gpu, "q8_0", "q4_g64", d, H, n - 1, k[:-1], v[:-1])
    q = torch.from_numpy(rng.standard_normal((1, hq, d)).astype(np.float32)).to(gpu)
    lens = torch.tensor([n], device=gpu)
    st = torch.zeros(1, dtype=torch.int32, device=gpu)
    L2 = Layer.create("q8_0", "q4_g64", d, H, 1, (n + 31) // 32 * 32, device=gpu)
    append_rows(L2, torch.from_numpy(k[:-1]).to(gpu), torch.from_numpy(v[:-1]).to(gpu), 0, 0)
    kvq_append_attend_decode(L2, torch.from_numpy(k[-1:]).to(gpu), torch.from_numpy(v[-1:]).to(gpu), q, lens, n,
                             0.1, dev_status=st)
    assert st.item() == 0  # an ordinary new row: nothing stored
    big = (v[-1:] * 1e5).astype(np.float32)
    kvq_append_attend_decode(L2, torch.from_numpy(k[-1:]).to(gpu), torch.from_numpy(big).to(gpu), q, lens, n, 0.1,
                             dev_status=st)
    assert st.item() == KVQ_EOVERFLOW


def _prefill(gpu, kmul, vmul, seed):
    rng = np.random.default_rng(seed)
    d, H, hq, P, T = 128, 2, 8, 150, 40
    n = P + T
    k = rng.standard_normal((n, H, d)).astype(np.float32)
    v = rng.standard_normal((n, H, d)).astype(np.float32)
    k[64:96] = np.clip(k[64:96], -4.5, 4.5) * kmul
    v[96:128] = np.clip(v[96:128], -4.5, 4.5) * vmul
    L = _layer(gpu, "q8_0", "q4_0", d, H, n, k, v)
    q = torch.from_numpy(rng.standard_normal((T, hq, d)).astype(np.float32)).to(gpu).to(torch.bfloat16)
    st = torch.zeros(1, dtype=torch.int32, device=gpu)
    out = kvq_attend_prefill(L, q, 0, P, 1 / np.sqrt(d), dev_status=st).cpu().numpy()
    kh = oracle.quant_dequant("q8_0", np.ascontiguousarray(k.transpose(1, 0, 2)))
    vh = oracle.quant_dequant("q4_0", np.ascontiguousarray(v.transpose(1, 0, 2)))
    ref = oracle.attend_prefill(q.float().cpu().numpy(), kh, vh, P, 1 / np.sqrt(d))
    return int(st.item()), out, ref


def test_prefill_values_inside_the_range_match(gpu):
    # large values (|v| up to 54000), ordinary keys: no report, the oracle's result.
    # (Keys of that size would put the scores near 1e4, where the binary16
    # rounding of K_hat moves a score by several units: a precision limit of
    # binary16 keys, not of the range.)
    status, out, ref = _prefill(gpu, 1.0, 12000.0, seed=5)
    assert status == 0
    assert np.isfinite(out).all() and rel_err(out, ref) <= 1e-2
    status, _, _ = _prefill(gpu, 12000.0, 1.0, seed=8)
    assert status == 0  # keys inside the range are not reported either


@pytest.mark.parametrize("kmul,vmul", [(1e5, 1.0), (1.0, 1e5)])
def test_prefill_values_beyond_the_range_are_reported(gpu, kmul, vmul):
    status, _, _ = _prefill(gpu, kmul, vmul, seed=6)
    assert status == KVQ_EOVERFLOW


def test_status_untouched_for_ordinary_calls(gpu):
    status, out, ref = _decode(gpu, "q4_g64", "q4_g64", 1.0, 1.0, seed=7)
    assert status == 0 and rel_err(out, ref) <= 1e-3
