"""CPU checks of the HIP library's host side: the C-ABI library loads and
exports every symbol include/kvq.h declares, host-only sizing, argument
validation (which returns before anything touches a GPU), and the in-block
permutation used by the planes."""
import ctypes
import glob
import os
import re

import numpy as np
import pytest

from block_quantized_kv_amd import _binding as B
from block_quantized_kv_amd import layout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def _declared_functions(header):
    text = re.sub(r"/\*.*?\*/", "", open(header).read(), flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z0-9_]+)\s*\(", text)))


def _library_of(header):
    """kvq_probe.h is exported by the measurement library, every other header by libkvq.so."""
    if os.path.basename(header) == "kvq_probe.h":
        from block_quantized_kv_amd import probe
        return probe.load_probe_library()
    return B.load_library()


def test_library_exports_every_declared_symbol():
    seen = set()
    for h in HEADERS:
        lib = _library_of(h)
        for n in _declared_functions(h):
            assert hasattr(lib, n), (os.path.basename(h), n)
            seen.add(n)
    assert {"kvq_append", "kvq_attend_decode", "kvq_attend_prefill", "kvq_dequant",
            "kvq_append_attend_decode", "kvq_probe_stream_read", "kvq_probe_mfma_f16"} <= seen


def test_probes_are_not_in_the_attention_library():
    lib = B.load_library()
    for n in ("kvq_probe_stream_read", "kvq_probe_mfma_f16"):
        assert not hasattr(lib, n), n


@pytest.mark.parametrize("codec,bpv", [("q4_g64", 4.25), ("q4_0", 4.5), ("q8_0", 8.5)])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_plane_bytes_bits_per_value(codec, bpv, d):
    # den_llama.cpp, "What this fork is": Q4_G64 is 4.25 bits per value.
    c, s = B.kvq_plane_bytes(codec, d, 4, 2, 1024)
    assert (c + s) * 8 == bpv * 4 * 2 * 1024 * d
    assert B.kvq_row_code_bytes(codec, d) == (d if codec == "q8_0" else d // 2)


def test_plane_bytes_decode_config_sizes():
    # One K plane of the 64K-context Q4_G64 workload: 65536 rows x 4 heads x 136 B.
    c, s = B.kvq_plane_bytes("q4_g64", 256, 4, 1, 65536)
    assert c + s == 35_651_584


def _fake_plane(codec="q8_0", role=0, d=128, heads=2, seqs=1, cap=64, codes=0x10000, scales=0x20000):
    return B._Plane(B.CODECS[codec], role, d, heads, seqs, 0, cap, codes, scales)


def _call_decode(L, q=0x1000, seq_len=0x2000, n_seqs=1, hq=4, max_len=64, out=0x3000, ws=0x4000,
                 ws_bytes=1 << 30):
    lib = B.load_library()
    return lib.kvq_attend_decode(ctypes.byref(L), q, seq_len, n_seqs, hq, max_len, 0.1, out, ws,
                                 ws_bytes, None, None)


def test_validation_errors_return_before_launch():
    lib = B.load_library()
    good = B._Layer(_fake_plane(role=0), _fake_plane(codec="q4_0", role=1, codes=0x30000, scales=0x40000))
    # decode: every failing argument -> exact status, nothing enqueued (no GPU here)
    assert lib.kvq_attend_decode(None, 1, 1, 1, 4, 64, 0.1, 1, 1, 1, None, None) == 1
    assert _call_decode(good, q=0) == 1
    assert _call_decode(good, q=0x1004) == 1                      # misaligned q
    assert _call_decode(good, hq=3) == 1                          # not a multiple of Hkv
    assert _call_decode(good, hq=2 * 17) == 2                     # GQA 17 > 16
    assert _call_decode(good, max_len=65) == 3                    # beyond capacity
    assert _call_decode(good, n_seqs=2) == 1                      # more than the plane holds
    assert _call_decode(good, ws_bytes=16) == 4                   # workspace too small
    assert _call_decode(good, ws=0) == 4
    bad_role = B._Layer(_fake_plane(role=1), good.v)
    assert _call_decode(bad_role) == 1
    bad_shape = B._Layer(good.k, _fake_plane(codec="q4_0", role=1, cap=96, codes=0x30000, scales=0x40000))
    assert _call_decode(bad_shape) == 1
    bad_d = B._Layer(_fake_plane(d=96), _fake_plane(role=1, d=96, codes=0x30000, scales=0x40000))
    assert _call_decode(bad_d) == 2
    bad_cap = B._Layer(_fake_plane(cap=40), _fake_plane(role=1, cap=40, codes=0x30000, scales=0x40000))
    assert _call_decode(bad_cap) == 1
    misaligned = B._Layer(_fake_plane(codes=0x10010), good.v)
    assert _call_decode(misaligned) == 1
    assert "aligned" in B.kvq_last_error()
    # append
    assert lib.kvq_append(ctypes.byref(good), 0, 0, 0x5000, 0x6000, 4, None, None) == 1
    assert lib.kvq_append(ctypes.byref(good), 0x7000, 0, 0x5000, 0x6000, -1, None, None) == 1
    assert lib.kvq_append(ctypes.byref(good), 0x7000, 0, 0, 0x6000, 4, None, None) == 1
    assert lib.kvq_append(ctypes.byref(good), 0x7000, 0, 0x5000, 0x6000, 0, None, None) == 0
    # prefill
    assert lib.kvq_attend_prefill(ctypes.byref(good), 0x1000, 0, 60, 8, 4, 0.1, 0x3000, 0, 0, None, None) == 3
    assert lib.kvq_attend_prefill(ctypes.byref(good), 0x1000, 1, 0, 8, 4, 0.1, 0x3000, 0, 0, None, None) == 1
    # more (token, head) columns than one launch holds: 2^21 tokens x 1024 q-heads per kv-head
    wide = B._Layer(_fake_plane(cap=1 << 22), _fake_plane(codec="q4_0", role=1, cap=1 << 22, codes=0x30000,
                                                          scales=0x40000))
    assert lib.kvq_attend_prefill(ctypes.byref(wide), 0x1000, 0, 0, 1 << 21, 2048, 0.1, 0x3000, 0, 0, None,
                                  None) == 2
    # dequant
    p = _fake_plane()
    assert lib.kvq_dequant(ctypes.byref(p), 0, 60, 8, 0x3000, None) == 3
    assert lib.kvq_dequant(ctypes.byref(p), 0, 0, 8, 0, None) == 1
    assert lib.kvq_dequant(ctypes.byref(p), 0, 0, 0, 0x3000, None) == 0
    assert B.kvq_status_str(4).startswith("KVQ_EWORKSPACE")


def test_multi_query_decode_validation():
    lib = B.load_library()
    good = B._Layer(_fake_plane(role=0), _fake_plane(codec="q4_0", role=1, codes=0x30000, scales=0x40000))

    def call(q_len, hq=4, ws_bytes=1 << 30):
        return lib.kvq_attend_decode_mq(ctypes.byref(good), 0x1000, 0x2000, 1, q_len, hq, 64, 0.1, 0x3000,
                                        0x4000, ws_bytes, None, None)
    assert call(0) == 1                 # no query
    assert call(65) == 1                # above KVQ_MAX_QUERIES
    assert call(2, hq=3) == 1           # not a multiple of Hkv
    assert call(2, ws_bytes=16) == 4    # workspace too small
    # the partials of one launch hold at most 16 / gqa queries: the workspace
    # grows with q_len up to that and no further (gqa 2 -> 8 queries)
    ws = [lib.kvq_decode_mq_workspace_bytes(ctypes.byref(good), 4, 1, n, 64) for n in (1, 2, 8, 9, 64)]
    assert ws[0] == lib.kvq_decode_workspace_bytes(ctypes.byref(good), 4, 1, 64)
    assert ws[0] < ws[1] < ws[2] == ws[3] == ws[4]


def test_fused_append_decode_validation():
    # every call here must fail in argument checking (the pointers are fake)
    lib = B.load_library()
    good = B._Layer(_fake_plane(role=0), _fake_plane(codec="q4_0", role=1, codes=0x30000, scales=0x40000))

    def call(k, v, ws_bytes=1 << 30, q=0x1000):
        return lib.kvq_append_attend_decode(ctypes.byref(good), k, v, q, 0x2000, 1, 4, 64, 0.1, 0x3000,
                                            0x4000, ws_bytes, None, None)

    def call_mq(k, v, q_len):
        return lib.kvq_append_attend_decode_mq(ctypes.byref(good), k, v, 0x1000, 0x2000, 1, q_len, 4, 64, 0.1,
                                               0x3000, 0x4000, 1 << 30, None, None)
    assert call(None, 0x5000) == 1          # k_new missing
    assert call(0x5000, None) == 1          # v_new missing
    assert call(0x5004, 0x6000) == 1        # k_new not 16-byte aligned
    assert call(0x5000, 0x6008) == 1        # v_new not 16-byte aligned
    assert call(0x5000, 0x6000, q=0) == 1   # no query
    assert call(0x5000, 0x6000, ws_bytes=16) == 4
    assert call_mq(None, 0x6000, 2) == 1
    assert call_mq(0x5000, 0x6000, 0) == 1
    assert call_mq(0x5000, 0x6000, 65) == 1


def test_probe_validation():
    # sizes that do not split into whole 8 KiB stripes per wave are refused
    from block_quantized_kv_amd import probe
    lib = probe.load_probe_library()
    assert lib.kvq_probe_stream_read(None, 1 << 20, 8, 0x1000, None) == 1
    assert lib.kvq_probe_stream_read(0x10000, (1 << 20) + 4096, 8, 0x1000, None) == 1
    assert lib.kvq_probe_stream_read(0x10000, 1 << 20, 0, 0x1000, None) == 1
    assert lib.kvq_probe_stream_read(0x10000, 1 << 31, 8, 0x1000, None) == 1
    # the matrix-core loop refuses a null sink and non-positive sizes
    assert lib.kvq_probe_mfma_f16(256, 100, None, None, None) == 1
    assert lib.kvq_probe_mfma_f16(0, 100, 0x1000, None, None) == 1
    assert lib.kvq_probe_mfma_f16(256, 0, 0x1000, None, None) == 1


def test_decode_workspace_grows_with_length():
    good = B._Layer(_fake_plane(cap=1 << 17), _fake_plane(role=1, cap=1 << 17, codes=0x30000, scales=0x40000))
    lib = B.load_library()
    a = lib.kvq_decode_workspace_bytes(ctypes.byref(good), 4, 1, 1024)
    b = lib.kvq_decode_workspace_bytes(ctypes.byref(good), 4, 1, 1 << 17)
    assert 0 < a <= b


@pytest.mark.parametrize("codec", ["q8_0", "q4_0", "q4_g64", "f16"])
@pytest.mark.parametrize("role", ["k", "v"])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_block_permutation_is_a_bijection(codec, role, d):
    byte, shift = layout.code_positions(codec, role, d)
    rb = layout.row_bytes(codec, d)
    if codec == "f16":  # a value's two bytes: its low byte sits at an even offset
        assert (byte % 2 == 0).all()
        slot = byte // 2
        n_slots = 32 * rb // 2
    else:
        slot = byte * 2 + shift // 4 if codec != "q8_0" else byte
        n_slots = 32 * rb * (2 if codec != "q8_0" else 1)
    assert slot.min() == 0 and slot.max() == n_slots - 1
    assert np.unique(slot).size == slot.size == n_slots
    sidx = layout.scale_positions(codec, role, d)
    assert np.unique(sidx).size == sidx.size == 32 * layout.n_scales(codec, d)


def test_unpack_inverts_a_scatter_f16():
    d, nb = 128, 2
    rng = np.random.default_rng(1)
    for role in ("k", "v"):
        rows = rng.integers(0, 256, size=(nb * 32, 2 * d), dtype=np.uint8)
        byte, _ = layout.code_positions("f16", role, d)
        blocks = np.zeros((nb, 32 * 2 * d), np.uint8)
        for bi in range(nb):
            for j in range(32):
                for c in range(d):
                    blocks[bi, byte[j, c]] = rows[bi * 32 + j, 2 * c]
                    blocks[bi, byte[j, c] + 1] = rows[bi * 32 + j, 2 * c + 1]
        assert np.array_equal(layout.unpack_codes("f16", role, d, blocks), rows)


def test_f16_control_codec_sizes_and_pairing():
    # 16 bits per value, no scales
    c, sc = B.kvq_plane_bytes("f16", 128, 8, 1, 1024)
    assert sc == 0 and c * 8 == 16 * 8 * 1024 * 128 and B.kvq_row_code_bytes("f16", 256) == 512
    lib = B.load_library()
    f16 = lambda role, d=128, codes=0x10000: _fake_plane(codec="f16", role=role, d=d, codes=codes, scales=0)
    both = B._Layer(f16(0), f16(1, codes=0x30000))
    # an f16 plane needs no scales pointer: validation passes up to the workspace check
    assert _call_decode(both, ws_bytes=16) == 4
    # f16 pairs only with f16 (append, decode); decode reads it at head_dim <= 128; prefill not at all
    mixed = B._Layer(f16(0), _fake_plane(codec="q4_0", role=1, codes=0x30000, scales=0x40000))
    assert _call_decode(mixed) == 2
    assert lib.kvq_append(ctypes.byref(mixed), 0x5000, 0x6000, 0x1000, 0x2000, 4, None, None) == 2
    wide = B._Layer(f16(0, d=256), f16(1, d=256, codes=0x30000))
    assert _call_decode(wide) == 2
    assert lib.kvq_attend_prefill(ctypes.byref(both), 0x1000, 0, 0, 16, 4, 0.1, 0x3000, None, 0, None, None) == 2


@pytest.mark.parametrize("codec", ["q8_0", "q4_0", "q4_g64"])
@pytest.mark.parametrize("role", ["k", "v"])
def test_unpack_inverts_a_scatter(codec, role):
    d, nb = 128, 3
    rng = np.random.default_rng(0)
    rb = layout.row_bytes(codec, d)
    rows = rng.integers(0, 256, size=(nb * 32, rb), dtype=np.uint8)
    # scatter row-major codes into blocks with the documented positions
    byte, shift = layout.code_positions(codec, role, d)
    blocks = np.zeros((nb, 32 * rb), np.uint8)
    for bi in range(nb):
        for j in range(32):
            r = rows[bi * 32 + j]
            for c in range(d):
                v = r[c] if codec == "q8_0" else (r[c // 2] >> (4 * (c % 2))) & 0xF
                blocks[bi, byte[j, c]] |= np.uint8(v << shift[j, c])
    back = layout.unpack_codes(codec, role, d, blocks)
    assert np.array_equal(back, rows)


def test_noalloc_size_check_runs_before_the_device():
    # a call whose partials exceed the library's scratch is refused on the
    # host (KVQ_EWORKSPACE), before the scratch is looked up on any GPU
    lib = B.load_library()
    assert lib.kvq_noalloc_scratch_bytes() == 16 << 20
    big = B._Layer(_fake_plane(heads=8, seqs=64, cap=131072),
                   _fake_plane(codec="q4_0", role=1, heads=8, seqs=64, cap=131072, codes=0x30000, scales=0x40000))
    st = lib.kvq_append_attend_decode_noalloc(ctypes.byref(big), 0x5000, 0x6000, 0x1000, 0x2000, 64, 32, 131072,
                                              0.1, 0x3000, None, None)
    assert st == 4 and b"no-allocation" in lib.kvq_last_error()
    # argument errors are still reported first
    assert lib.kvq_append_attend_decode_noalloc(ctypes.byref(big), None, 0x6000, 0x1000, 0x2000, 1, 32, 64, 0.1,
                                                0x3000, None, None) == 1


def test_paged_prefill_validation():
    lib = B.load_library()
    pool = B._Layer(_fake_plane(cap=64, seqs=8), _fake_plane(codec="q4_0", role=1, cap=64, seqs=8, codes=0x30000,
                                                             scales=0x40000))
    P = B._PagedLayer(pool, 0x7000, 2, 4)   # 2 sequences x 4 pages of 64 rows
    call = lambda seq=0, pos0=0, T=16, hq=4, q=0x1000, out=0x3000: lib.kvq_paged_attend_prefill(
        ctypes.byref(P), q, seq, pos0, T, hq, 0.1, out, None, 0, None, None)
    assert call(seq=2) == 1                      # only 2 sequences in the table
    assert call(pos0=250, T=7) == 3              # past 4 pages x 64 rows
    assert call(q=0) == 1
    assert call(hq=3) == 1
    assert call(T=0) == 0                        # nothing to do
    bad = B._PagedLayer(pool, 0, 2, 4)
    assert lib.kvq_paged_attend_prefill(ctypes.byref(bad), 0x1000, 0, 0, 16, 4, 0.1, 0x3000, None, 0, None,
                                        None) == 1
    # more pages than a paged prefill addresses
    big = B._PagedLayer(B._Layer(_fake_plane(cap=32, seqs=8), _fake_plane(codec="q4_0", role=1, cap=32, seqs=8,
                                                                          codes=0x30000, scales=0x40000)),
                        0x7000, 1, 10000)
    assert lib.kvq_paged_attend_prefill(ctypes.byref(big), 0x1000, 0, 200000, 16, 4, 0.1, 0x3000, None, 0, None,
                                        None) == 2


def test_debug_append_wait_validation():
    lib = B.load_library()
    assert lib.kvq_debug_append_wait(-1, 0) == 1
    assert lib.kvq_debug_append_wait(1 << 20, 0) == 0


def test_plain_c_example_is_built_and_starts():
    """The plain-C user of the C ABI (tests/c_abi/decode_step.c) is built with
    the libraries and links against libkvq.so; without arguments it prints its
    usage and exits before touching a GPU."""
    import subprocess
    from block_quantized_kv_amd import build
    assert os.path.exists(build.C_EXAMPLE_BIN), "build it with block_quantized_kv_amd/build.py"
    r = subprocess.run([build.C_EXAMPLE_BIN], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "usage" in r.stderr


def test_binding_rejects_tensors_on_another_device():
    """Every tensor of a call must sit on the cache's device; the binding
    refuses a mix before anything reaches the library (here a cache held in
    host memory and queries on the meta device, so no GPU is needed)."""
    import torch
    layer = B.Layer.create("q8_0", "q4_0", 64, 1, 1, 32, device="cpu")
    q = torch.empty(1, 4, 64, device="meta")
    lens = torch.empty(1, dtype=torch.int64, device="meta")
    with pytest.raises(ValueError, match="cache is on"):
        B.kvq_attend_decode(layer, q, lens, 32, 0.1)
    with pytest.raises(ValueError, match="cache is on"):
        B.kvq_append(layer, torch.empty(1, 1, 64, device="meta"), None, torch.zeros(1, dtype=torch.int32),
                     torch.zeros(1, dtype=torch.int64))
