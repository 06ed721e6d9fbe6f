"""The C ABI used from a plain C program, with no Python in between
(tests/c_abi/decode_step.c, built by block_quantized_kv_amd/build.py): it
builds a cache with kvq_append and runs one kvq_append_attend_decode step,
the way a serving loop written in C would; its output is compared with the
oracle at the decode bar (max|gpu - oracle| / max|oracle| <= 1e-3), and both
device status words must stay 0."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from gpu_helpers import rel_err

pytestmark = pytest.mark.gpu
BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "decode_step")
CODEC_IDS = {"q8_0": 0, "q4_0": 1, "q4_g64": 2, "f16": 3}


@pytest.mark.parametrize("kc,vc,d,hkv,hq,n", [
    ("q8_0", "q4_g64", 64, 1, 4, 256),      # the tiny decode configuration's shape
    ("q8_0", "q4_0", 128, 8, 32, 3001),     # ragged tail, several splits
    ("q4_g64", "q4_g64", 256, 4, 24, 5000),
    ("f16", "f16", 128, 2, 8, 777),         # the f16 control codec
])
def test_c_program_decode_step(gpu, tmp_path, kc, vc, d, hkv, hq, n):
    if not os.path.exists(BIN):
        pytest.fail(f"{BIN} is missing: build it with block_quantized_kv_amd/build.py")
    rng = np.random.default_rng(n + d)
    k = rng.standard_normal((n, hkv, d)).astype(np.float32)
    v = rng.standard_normal((n, hkv, d)).astype(np.float32)
    q = rng.standard_normal((hq, d)).astype(np.float32)
    k.tofile(tmp_path / "k.f32")
    v.tofile(tmp_path / "v.f32")
    q.tofile(tmp_path / "q.f32")
    scale = float(np.float32(1.0 / np.sqrt(d)))
    r = subprocess.run([BIN, str(tmp_path), str(CODEC_IDS[kc]), str(CODEC_IDS[vc]), str(d), str(hkv), str(hq),
                        str(n), repr(scale)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert "append status 0, decode status 0" in r.stdout
    out = np.fromfile(tmp_path / "out.f32", dtype=np.float32).reshape(hq, d)
    kh = oracle.quant_dequant(kc, np.ascontiguousarray(k.transpose(1, 0, 2)))
    vh = oracle.quant_dequant(vc, np.ascontiguousarray(v.transpose(1, 0, 2)))
    ref = oracle.attend_decode(q, kh, vh, n, scale)
    assert rel_err(out, ref) <= 1e-3
