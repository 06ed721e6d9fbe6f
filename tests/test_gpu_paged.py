"""GPU parity of the paged planes (a page pool addressed through a block table).

A paged layer must hold, page by page, exactly the bytes a contiguous layer
holds for the same rows (kvq_paged_append against kvq_append), and attention
over it must return what attention over the contiguous layer returns: to
5e-4 of max|out| (the waves of a split take blocks in whatever order they
get them, which moves the binary16 rounding of the probabilities), and
within the decode bar of the oracle, 1e-3 of max|oracle|.

Covered: pages of 32, 64, 96, 160, 256 and 2048 rows (96 and 160: not powers of two,
so the page lookup divides); pages shuffled over a pool
larger than needed; ragged lengths (a length inside a page, on a page
boundary, shorter than a page); several sequences; one and two queries per
sequence; the fused append + decode through the table; a table entry outside
the pool (the append reports KVQ_ERANGE and skips the row, the attention
stays finite); the 64K-context Q4_G64 step on 256-row pages; and chunked
prefill through the table (below).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from block_quantized_kv_amd import (Layer, PagedLayer, kvq_append, kvq_attend_decode_mq, kvq_paged_append,
                                    kvq_paged_append_attend_decode_mq, kvq_paged_attend_decode_mq, layout)
from gpu_helpers import append_rows, rel_err

pytestmark = pytest.mark.gpu
TOL = 1e-3
SAME = 5e-4


def _pool_for(kc, vc, d, hkv, n_seqs, max_pages, page_rows, gpu, seed, spare=3):
    """A pool with n_seqs * max_pages + spare pages and a table that scatters them."""
    n_pages = n_seqs * max_pages + spare
    perm = np.random.default_rng(seed).permutation(n_pages)[: n_seqs * max_pages]
    table = torch.from_numpy(perm.reshape(n_seqs, max_pages).astype(np.int32)).to(gpu)
    pool = Layer.create(kc, vc, d, hkv, n_pages, page_rows, device=gpu)
    return PagedLayer(pool, table)


def _paged_rows(pl, seq, k_rows, v_rows, row0=0):
    n = k_rows.shape[0]
    dev = k_rows.device
    for a in range(0, n, 16384):
        b = min(n, a + 16384)
        kvq_paged_append(pl, k_rows[a:b].contiguous(), v_rows[a:b].contiguous(),
                         torch.full((b - a,), seq, dtype=torch.int32, device=dev),
                         torch.arange(row0 + a, row0 + b, dtype=torch.int64, device=dev))


def _same_pages(pl: PagedLayer, contig: Layer, n_used_pages):
    """Page i of sequence b in the pool holds the bytes of rows [i*R, (i+1)*R)."""
    R = pl.page_rows
    table = pl.block_table.cpu().numpy()
    for ppool, pc, name in ((pl.pool.k, contig.k, "K"), (pl.pool.v, contig.v, "V")):
        H = pc.n_kv_heads
        cb = 32 * layout.row_bytes(pc.codec, pc.head_dim)          # code bytes per 32-row block
        sb = 32 * pc.head_dim // layout.GROUP[pc.codec]            # binary16 scales per block
        pool_c = ppool.codes.view(ppool.n_seqs, H, R // 32, cb)
        pool_s = ppool.scales.view(ppool.n_seqs, H, R // 32, sb)
        con_c = pc.codes.view(pc.n_seqs, H, pc.capacity // 32, cb)
        con_s = pc.scales.view(pc.n_seqs, H, pc.capacity // 32, sb)
        for b, n_pages in enumerate(n_used_pages):
            for i in range(n_pages):
                pg = int(table[b, i])
                blk = slice(i * R // 32, (i + 1) * R // 32)
                assert torch.equal(pool_c[pg], con_c[b, :, blk]), (name, "codes", b, i)
                assert torch.equal(pool_s[pg], con_s[b, :, blk]), (name, "scales", b, i)


def _case(gpu, kc, vc, d, hq, hkv, lens, page_rows, q_len=1, seed=0, fused=False, oracle_check=True):
    rng = np.random.default_rng(seed)
    S = len(lens)
    max_pages = max(1, -(-max(lens) // page_rows))
    cap = max_pages * page_rows
    pl = _pool_for(kc, vc, d, hkv, S, max_pages, page_rows, gpu, seed)
    contig = Layer.create(kc, vc, d, hkv, S, cap, device=gpu)
    k = rng.standard_normal((S, cap, hkv, d)).astype(np.float32)
    v = rng.standard_normal((S, cap, hkv, d)).astype(np.float32)
    q = rng.standard_normal((S, q_len, hq, d)).astype(np.float32)
    for s, n in enumerate(lens):
        old = max(n - q_len, 0) if fused else n
        if old:
            kt, vt = torch.from_numpy(k[s, :old]).to(gpu), torch.from_numpy(v[s, :old]).to(gpu)
            append_rows(contig, kt, vt, s, 0)
            _paged_rows(pl, s, kt, vt)
    lens_t = torch.tensor(lens, dtype=torch.int64, device=gpu)
    scale = 1.0 / np.sqrt(d)
    ml = max(max(lens), 1)
    qd = torch.from_numpy(q).to(gpu)
    if fused:
        # new rows: entry i of sequence s is row lens[s] - q_len + i (zeros at
        # negative positions, which are skipped); the contiguous layer gets
        # them through kvq_append
        kn = np.zeros((S, q_len, hkv, d), np.float32)
        vn = np.zeros((S, q_len, hkv, d), np.float32)
        sq, pos, rk, rv = [], [], [], []
        for s, n in enumerate(lens):
            for i in range(q_len):
                p = n - q_len + i
                if p >= 0:
                    kn[s, i], vn[s, i] = k[s, p], v[s, p]
                    sq.append(s)
                    pos.append(p)
                    rk.append(k[s, p])
                    rv.append(v[s, p])
        if sq:
            kvq_append(contig, torch.from_numpy(np.stack(rk)).to(gpu), torch.from_numpy(np.stack(rv)).to(gpu),
                       torch.tensor(sq, dtype=torch.int32, device=gpu), torch.tensor(pos, dtype=torch.int64, device=gpu))
        out = kvq_paged_append_attend_decode_mq(pl, torch.from_numpy(kn).to(gpu), torch.from_numpy(vn).to(gpu), qd,
                                                lens_t, ml, scale).cpu().numpy()
    else:
        out = kvq_paged_attend_decode_mq(pl, qd, lens_t, ml, scale).cpu().numpy()
    ref_out = kvq_attend_decode_mq(contig, qd, lens_t, ml, scale).cpu().numpy()
    _same_pages(pl, contig, [-(-n // page_rows) for n in lens])
    assert np.isfinite(out).all()
    if np.abs(ref_out).max() > 0:
        assert rel_err(out, ref_out) <= SAME
    if oracle_check:
        for s, n in enumerate(lens):
            kh = oracle.quant_dequant(kc, np.ascontiguousarray(k[s].transpose(1, 0, 2)))
            vh = oracle.quant_dequant(vc, np.ascontiguousarray(v[s].transpose(1, 0, 2)))
            for i in range(q_len):
                rows = n - q_len + i + 1
                if rows <= 0:
                    assert np.array_equal(out[s, i], np.zeros_like(out[s, i]))
                    continue
                ref = oracle.attend_decode(q[s, i], kh, vh, rows, scale)
                assert rel_err(out[s, i], ref) <= TOL, (kc, vc, d, n, page_rows, q_len, i)


@pytest.mark.parametrize("page_rows", [32, 64, 96, 160, 256, 2048])  # 96, 160: not powers of two
def test_page_sizes(gpu, page_rows):
    _case(gpu, "q4_g64", "q4_0", 128, hq=8, hkv=2, lens=[1500, 700], page_rows=page_rows, seed=page_rows)


@pytest.mark.parametrize("kc,vc,d", [("q8_0", "q4_0", 128), ("q4_g64", "q4_g64", 256), ("q8_0", "q4_0", 256),
                                     ("q8_0", "q8_0", 64), ("q4_0", "q4_g64", 64)])
def test_codec_pairs(gpu, kc, vc, d):
    _case(gpu, kc, vc, d, hq=12, hkv=2, lens=[640, 65, 1], page_rows=64, seed=d + len(kc))


def test_ragged_lengths(gpu):
    # inside a page, on a page boundary, shorter than one page, several splits
    _case(gpu, "q8_0", "q4_0", 64, hq=4, hkv=1, lens=[257, 512, 31, 9000], page_rows=256, seed=3)


def test_two_queries(gpu):
    _case(gpu, "q4_g64", "q8_0", 128, hq=8, hkv=2, lens=[700, 257], page_rows=64, q_len=2, seed=4)


@pytest.mark.parametrize("q_len,lens", [(1, [700, 257, 1]), (2, [257, 65]), (3, [2, 300])])
def test_fused_append(gpu, q_len, lens):
    _case(gpu, "q4_0", "q4_g64", 128, hq=8, hkv=2, lens=lens, page_rows=64, q_len=q_len, seed=q_len + 10,
          fused=True)


@pytest.mark.parametrize("kc,vc", [("q4_g64", "q4_g64"), ("q8_0", "q4_0")])
def test_fused_append_head_dim_256(gpu, kc, vc):
    # the 64K model's head size through pages, two new rows per sequence
    _case(gpu, kc, vc, 256, hq=12, hkv=2, lens=[1100, 33], page_rows=64, q_len=2, seed=len(kc) + 40, fused=True)


def test_entry_outside_the_pool(gpu):
    # a table entry of -1 inside the length: the append reports KVQ_ERANGE and
    # writes nothing for those rows; the attention reads zeros for them and
    # stays finite
    pl = _pool_for("q8_0", "q4_0", 64, 1, 1, 4, 32, gpu, seed=5, spare=0)
    pl.block_table[0, 2] = -1
    rng = np.random.default_rng(5)
    k = torch.from_numpy(rng.standard_normal((128, 1, 64)).astype(np.float32)).to(gpu)
    v = torch.from_numpy(rng.standard_normal((128, 1, 64)).astype(np.float32)).to(gpu)
    before = (pl.pool.k.codes.clone(), pl.pool.v.codes.clone())
    status = torch.zeros(1, dtype=torch.int32, device=gpu)
    kvq_paged_append(pl, k, v, torch.zeros(128, dtype=torch.int32, device=gpu),
                     torch.arange(128, dtype=torch.int64, device=gpu), dev_status=status)
    assert int(status.item()) == 3
    # every page the table names was written, none other
    written = [int(x) for x in pl.block_table[0].cpu().numpy() if x >= 0]
    for plane, old in ((pl.pool.k, before[0]), (pl.pool.v, before[1])):
        per_page = plane.codes.numel() // plane.n_seqs
        for pg in range(plane.n_seqs):
            same = torch.equal(plane.codes[pg * per_page:(pg + 1) * per_page], old[pg * per_page:(pg + 1) * per_page])
            assert same == (pg not in written), pg
    q = torch.from_numpy(rng.standard_normal((1, 1, 4, 64)).astype(np.float32)).to(gpu)
    out = kvq_paged_attend_decode_mq(pl, q, torch.tensor([128], dtype=torch.int64, device=gpu), 128, 0.125)
    assert torch.isfinite(out).all()


def test_workload_64k_on_256_row_pages(gpu):
    """The 64K-context Q4_G64 step on 256 shuffled 256-row pages, fused,
    against the same step on contiguous planes."""
    cfg = workloads.DECODE_64K
    n, H, d = cfg.ctx, cfg.n_kv_heads, cfg.head_dim
    kc, vc = cfg.layers[0]
    pl = _pool_for(kc, vc, d, H, 1, n // 256, 256, gpu, seed=64)
    contig = Layer.create(kc, vc, d, H, 1, cfg.capacity, device=gpu)
    k = workloads.kv_rows(cfg, 0, 0, "k", 0, n, gpu)
    v = workloads.kv_rows(cfg, 0, 0, "v", 0, n, gpu)
    append_rows(contig, k, v, 0, 0)
    _paged_rows(pl, 0, k[: n - 1], v[: n - 1])
    q = workloads.queries(cfg, 0, gpu)[:, None].contiguous()
    lens = torch.tensor([n], dtype=torch.int64, device=gpu)
    out = kvq_paged_append_attend_decode_mq(pl, k[n - 1:][None].contiguous(), v[n - 1:][None].contiguous(), q,
                                            lens, n, cfg.scale)
    ref = kvq_attend_decode_mq(contig, q, lens, n, cfg.scale)
    _same_pages(pl, contig, [n // 256])
    assert torch.isfinite(out).all()
    assert rel_err(out.cpu().numpy(), ref.cpu().numpy()) <= SAME


# ---- chunked prefill through the table ---------------------------------------------
# The prefill kernel reads a tile's blocks in a fixed order, so over paged
# planes holding the same rows it must return exactly what it returns over
# contiguous planes (bit for bit), and within the prefill bar of the oracle,
# 1e-2 of max|oracle|.

PTOL = 1e-2


def _prefill_case(gpu, kc, vc, d, hq, hkv, P, T, page_rows, seed, seqs=1, seq=0, bad_page=None):
    from block_quantized_kv_amd import kvq_attend_prefill, kvq_paged_attend_prefill
    n = P + T
    max_pages = (n + page_rows - 1) // page_rows + 1
    pl = _pool_for(kc, vc, d, hkv, seqs, max_pages, page_rows, gpu, seed)
    contig = Layer.create(kc, vc, d, hkv, seqs, max_pages * page_rows, device=gpu)
    rows = {}
    for s in range(seqs):
        q, k, v = workloads.prefill_inputs(gpu, seed_layer=seed + s, prefix=P, chunk=T, n_q_heads=hq,
                                           n_kv_heads=hkv, head_dim=d)
        _paged_rows(pl, s, k, v)
        append_rows(contig, k, v, s, 0)
        rows[s] = (q, k, v)
    q, k, v = rows[seq]
    kh = oracle.quant_dequant(kc, k.cpu().numpy().transpose(1, 0, 2).copy())
    vh = oracle.quant_dequant(vc, v.cpu().numpy().transpose(1, 0, 2).copy())
    if bad_page is not None:
        # a table entry outside the pool: those rows read as zeros
        table = pl.block_table.clone()
        table[seq, bad_page] = pl.pool.k.n_seqs + 5
        pl = PagedLayer(pl.pool, table)
        lo, hi = bad_page * page_rows, min(n, (bad_page + 1) * page_rows)
        kh[:, lo:hi] = 0.0
        vh[:, lo:hi] = 0.0
    scale = 1.0 / np.sqrt(d)
    out = kvq_paged_attend_prefill(pl, q, seq, P, scale).cpu().numpy()
    assert np.isfinite(out).all()
    if bad_page is None:
        ref_c = kvq_attend_prefill(contig, q, seq, P, scale).cpu().numpy()
        assert np.array_equal(out, ref_c)
    ref = oracle.attend_prefill(q.float().cpu().numpy(), kh, vh, P, scale)
    err = rel_err(out, ref)
    assert err <= PTOL, (kc, vc, d, P, T, page_rows, err)


@pytest.mark.parametrize("page_rows", [32, 64, 96, 256])  # 96: not a power of two
@pytest.mark.parametrize("kc,vc,d", [("q8_0", "q4_0", 128), ("q4_g64", "q4_g64", 256), ("q8_0", "q4_0", 256),
                                     ("q4_0", "q8_0", 64)])
def test_paged_prefill_matches_contiguous(gpu, kc, vc, d, page_rows):
    _prefill_case(gpu, kc, vc, d, 8, 2, 300, 77, page_rows, seed=page_rows + d)


@pytest.mark.parametrize("P,T", [(0, 1), (31, 33), (64, 64), (500, 260)])
def test_paged_prefill_ragged(gpu, P, T):
    _prefill_case(gpu, "q8_0", "q4_g64", 128, 6, 1, P, T, 64, seed=P + T)


def test_paged_prefill_middle_sequence(gpu):
    _prefill_case(gpu, "q4_0", "q4_0", 128, 8, 2, 200, 150, 32, seed=3, seqs=3, seq=1)


def test_paged_prefill_entry_outside_pool_reads_zeros(gpu):
    _prefill_case(gpu, "q8_0", "q4_0", 128, 8, 2, 300, 70, 64, seed=8, bad_page=2)


def test_paged_prefill_workload_2048_over_32768(gpu):
    """The chunked-prefill workload on 256-row pages shuffled over the pool:
    bit for bit what the contiguous planes give; 256 rows against the oracle."""
    from block_quantized_kv_amd import kvq_attend_prefill, kvq_paged_attend_prefill
    W = workloads.PREFILL
    P, T, hq, hkv, d = W["prefix"], W["chunk"], W["n_q_heads"], W["n_kv_heads"], W["head_dim"]
    kc, vc = W["k_codec"], W["v_codec"]
    page_rows = 256
    max_pages = (P + T) // page_rows
    pl = _pool_for(kc, vc, d, hkv, 1, max_pages, page_rows, gpu, seed=21)
    contig = Layer.create(kc, vc, d, hkv, 1, P + T, device=gpu)
    q, k, v = workloads.prefill_inputs(gpu)
    _paged_rows(pl, 0, k, v)
    append_rows(contig, k, v, 0, 0)
    scale = 1.0 / np.sqrt(d)
    out = kvq_paged_attend_prefill(pl, q, 0, P, scale).cpu().numpy()
    assert np.array_equal(out, kvq_attend_prefill(contig, q, 0, P, scale).cpu().numpy())
    rng = np.random.default_rng(4)
    toks, heads = rng.integers(0, T, 256).astype(np.int32), rng.integers(0, hq, 256).astype(np.int32)
    kh = oracle.quant_dequant(kc, k.cpu().numpy().transpose(1, 0, 2).copy())
    vh = oracle.quant_dequant(vc, v.cpu().numpy().transpose(1, 0, 2).copy())
    ref = oracle.attend_prefill(q.float().cpu().numpy(), kh, vh, P, scale, tokens=toks, heads=heads)
    assert rel_err(out[toks, heads], ref) <= PTOL
