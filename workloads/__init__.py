"""Seeded synthetic workloads for the parity tests and the benchmark.

This module only draws random inputs with the shapes and value structure of
the workloads; it contains none of the method's arithmetic (no quantization,
no attention).  Both the HIP path and the CPU oracle consume what it returns.

Workload recipe (den_llama.cpp serves a 27B model at 32K / 65K / 196K context
with a q8_0 K / q4_0 V cache and 2048-token micro-batches, "Results" and
"Quick start"; Q4_G64 and layer-wise split KV in "What this fork is").  Real
K/V activations are replaced by:
  TINY        : 1 seq, 4 q-heads / 1 kv-head, d 64, ctx 256, N(0,1); K q8_0, V Q4_G64, scale 1/8
  DECODE_32K  : 1 seq, 32/8, d 128, ctx 32768; N(0,1) with 10 of the 1024
                (kv-head, channel) pairs x8 on every row (1% outlier channels),
                drawn separately for K and V; K q8_0, V q4_0
  DECODE_64K  : 1 seq, 24/4, d 256, ctx 65536; N(0,1) * s[h,c], s = exp(U[ln 1/4, ln 4])
                per (kv-head, channel), independent for K and V; Q4_G64 / Q4_G64;
                65535 rows pre-filled, the step appends row 65535 and attends 65536
  DECODE_196K : 1 seq, 24/4, d 256, ctx 196608, 4 layers; layer 0 q8_0/q8_0,
                layers 1-3 Q4_G64/Q4_G64; N(0,1)
  BATCHED     : 16 seqs, 32/8, d 128, lengths U{4096..131072}; N(0,1); K q8_0, V q4_0
  PREFILL     : 1 seq, 32/8, d 128, prefix 32768 + chunk 2048; Q bf16(N(0,1)),
                K/V N(0,1) fp32; K q8_0, V q4_0
Every tensor comes from its own torch.Generator seeded from (the workload's
seed id, layer, stream), so any piece can be regenerated alone on any device.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Config:
    seed_id: int              # first component of every generator seed
    name: str
    n_seqs: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ctx: int                  # context (max length) per sequence
    layers: tuple             # ((k_codec, v_codec), ...)
    structure: str = "normal"  # normal | outliers | channel_scale
    append_step: bool = False  # timed step appends the last row before attending
    batched_lengths: bool = False
    extra: dict = field(default_factory=dict)

    @property
    def gqa(self):
        return self.n_q_heads // self.n_kv_heads

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def capacity(self):
        return (self.ctx + 31) // 32 * 32


TINY = Config(1, "tiny_decode_ctx256", 1, 4, 1, 64, 256, (("q8_0", "q4_g64"),))
DECODE_32K = Config(2, "decode_ctx32k_q8_0k_q4_0v", 1, 32, 8, 128, 32768, (("q8_0", "q4_0"),),
                    structure="outliers")
DECODE_64K = Config(3, "decode_ctx64k_q4g64", 1, 24, 4, 256, 65536, (("q4_g64", "q4_g64"),),
                    structure="channel_scale", append_step=True)
DECODE_196K = Config(4, "decode_ctx196k_split_kv_4layers", 1, 24, 4, 256, 196608,
                     (("q8_0", "q8_0"), ("q4_g64", "q4_g64"), ("q4_g64", "q4_g64"), ("q4_g64", "q4_g64")))
BATCHED = Config(5, "batched_decode_16seq_4k_128k", 16, 32, 8, 128, 131072, (("q8_0", "q4_0"),),
                 batched_lengths=True)
CONFIGS = {c.name: c for c in (TINY, DECODE_32K, DECODE_64K, DECODE_196K, BATCHED)}
PREFILL = dict(n_q_heads=32, n_kv_heads=8, head_dim=128, prefix=32768, chunk=2048,
               k_codec="q8_0", v_codec="q4_0")

# stream ids inside a workload
_Q, _K, _V, _AUX, _LEN, _QP = 1, 2, 3, 4, 5, 6


def _gen(device, seed_id, layer, stream, seq=0):
    g = torch.Generator(device=device)
    g.manual_seed(((seed_id * 131 + layer) * 1009 + stream) * 65537 + seq)
    return g


def seq_lengths(cfg: Config, device="cpu") -> torch.Tensor:
    """int64 [n_seqs] attended lengths."""
    if not cfg.batched_lengths:
        return torch.full((cfg.n_seqs,), cfg.ctx, dtype=torch.int64, device=device)
    g = _gen("cpu", cfg.seed_id, 0, _LEN)
    lens = torch.randint(4096, 131072 + 1, (cfg.n_seqs,), generator=g, dtype=torch.int64)
    return lens.to(device)


def queries(cfg: Config, layer: int, device) -> torch.Tensor:
    """fp32 [n_seqs][n_q_heads][head_dim] ~ N(0, 1)."""
    g = _gen(device, cfg.seed_id, layer, _Q)
    return torch.randn(cfg.n_seqs, cfg.n_q_heads, cfg.head_dim, generator=g, device=device)


def _structure(cfg: Config, layer: int, which: int, device) -> torch.Tensor | None:
    """Per-(kv-head, channel) multiplier [n_kv_heads][head_dim] or None."""
    g = _gen("cpu", cfg.seed_id, layer, _AUX * 10 + which)
    H, d = cfg.n_kv_heads, cfg.head_dim
    if cfg.structure == "outliers":
        n = max(1, round(0.01 * H * d))
        idx = torch.randperm(H * d, generator=g)[:n]
        m = torch.ones(H * d)
        m[idx] = 8.0
        return m.view(H, d).to(device)
    if cfg.structure == "channel_scale":
        u = torch.rand(H, d, generator=g, dtype=torch.float64)
        s = torch.exp(math.log(0.25) + u * (math.log(4.0) - math.log(0.25)))
        return s.to(torch.float32).to(device)
    return None


def kv_rows(cfg: Config, layer: int, seq: int, which: str, row0: int, n_rows: int, device):
    """fp32 [n_rows][n_kv_heads][head_dim] rows row0..row0+n_rows-1 of K or V
    (which = 'k' or 'v') of one sequence.  Rows are drawn in fixed chunks of
    4096 so any sub-range regenerates identically."""
    w = 0 if which == "k" else 1
    H, d = cfg.n_kv_heads, cfg.head_dim
    mult = _structure(cfg, layer, w, device)
    out = torch.empty(n_rows, H, d, device=device)
    CH = 4096
    c0, c1 = row0 // CH, (row0 + n_rows - 1) // CH if n_rows > 0 else row0 // CH - 1
    for ch in range(c0, c1 + 1):
        g = _gen(device, cfg.seed_id, layer, _K if w == 0 else _V, seq * 100003 + ch)
        blk = torch.randn(CH, H, d, generator=g, device=device)
        a, b = max(row0, ch * CH), min(row0 + n_rows, (ch + 1) * CH)
        out[a - row0:b - row0] = blk[a - ch * CH:b - ch * CH]
    if mult is not None:
        out *= mult
    return out


def prefill_inputs(device, seed_layer: int = 0, prefix: int | None = None, chunk: int | None = None,
                   n_q_heads: int | None = None, n_kv_heads: int | None = None,
                   head_dim: int | None = None):
    """(q bf16 [T][Hq][d], k fp32 [P+T][Hkv][d], v fp32 [P+T][Hkv][d]) for the
    chunked-prefill workload (sizes overridable for small parity cases)."""
    P = PREFILL["prefix"] if prefix is None else prefix
    T = PREFILL["chunk"] if chunk is None else chunk
    Hq = PREFILL["n_q_heads"] if n_q_heads is None else n_q_heads
    Hkv = PREFILL["n_kv_heads"] if n_kv_heads is None else n_kv_heads
    d = PREFILL["head_dim"] if head_dim is None else head_dim
    g = _gen(device, 50, seed_layer, _QP)
    q = torch.randn(T, Hq, d, generator=g, device=device).to(torch.bfloat16)
    g = _gen(device, 50, seed_layer, _K)
    k = torch.randn(P + T, Hkv, d, generator=g, device=device)
    g = _gen(device, 50, seed_layer, _V)
    v = torch.randn(P + T, Hkv, d, generator=g, device=device)
    return q, k, v
