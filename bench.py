#!/usr/bin/env python3
"""Benchmark: decode attention over a block-quantized KV cache on one MI355X.

Headline workload (metric "decode-attention effective KV GB/s @64K ctx"):
  one sequence, 24 query heads / 4 KV heads, head_dim 256, Q4_G64 K and V,
  context 65536.  One step appends the new token's K and V (row 65535) and
  attends over all 65536 rows -- the whole decode hot path (quantize-on-append,
  split-K attention, log-sum-exp combine) -- as one kvq_append_attend_decode
  call (the decode kernel writes the new row first).  The same step as two
  calls (kvq_append, then kvq_attend_decode) is timed beside it.
  The timed loop rotates over 16 independent caches (>= 1 GB in total) so
  the 256 MB last-level cache cannot serve the K/V bytes.

value = algorithmic bytes per step / step time, where the algorithmic bytes
are the quantized K+V bytes of every attended row read once per kv-head
(65536 x 4 x (136 + 136) B) plus the query, the output and the appended row
in/out.  Prefill (2048-token causal chunk over a 32768-token quantized prefix)
is reported beside it in TFLOP/s when its kernel is available.

Prints one JSON line.  Single GPU only: --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
ROTATE = 16
SETTLE_MS = 200.0   # untimed back-to-back work before each timed loop (see settle)


def settle(torch, fn, chunk: int, min_ms: float = SETTLE_MS) -> int:
    """Runs fn(i) back to back, untimed, synchronizing every `chunk` calls,
    until at least min_ms of wall time has passed; returns the call count.
    The GPU raises its clocks over the first tens of milliseconds of sustained
    work and lowers them again within half a second of idling (measured on
    this chip: the 2048-token prefill chunk takes ~1.5 ms per call at first and
    ~1.15 ms after ~40 ms of calls; the 64K decode step ~22.5 us at first and
    20.7-20.8 us after ~40 ms), so each timed loop starts from a GPU that has
    been busy for a while, as it is in serving.  `chunk` keeps the launch queue
    full between synchronizations."""
    t0 = time.perf_counter()
    i = 0
    while True:
        for _ in range(chunk):
            fn(i)
            i += 1
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= min_ms:
            return i


def _args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=500)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-quality", action="store_true")
    p.add_argument("--no-baselines", action="store_true")
    p.add_argument("--step-only", action="store_true",
                   help="time only the headline step (no two-call step, attention-only, multi-query, "
                        "baseline, prefill, quality or CPU legs): the run that profiles and counters use")
    p.add_argument("--prefill-only", action="store_true",
                   help="run only the prefill leg (2048-token chunk over a 32768-row prefix) and print its JSON: "
                        "the run that the prefill kernel's profile uses")
    p.add_argument("--write-busy-summary", nargs=2, metavar=("KERNEL", "PMC_DIR"),
                   help="summarize a rocprofv3 counter pass (KERNEL = prefill or decode) into profiles/ and exit")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run plain 256 MiB device copies (HBM counter calibration)")
    p.add_argument("--write-traffic-summary", nargs=2, metavar=("KERNEL", "PMC_DIR"),
                   help="summarize rocprofv3 FETCH_SIZE/WRITE_SIZE runs (PMC_DIR/{fetch,write,cfetch,cwrite}) of "
                        "KERNEL (decode or prefill) into profiles/ and exit")
    return p.parse_args()


# ---- counter-backed HBM traffic ---------------------------------------------
# rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) over this benchmark gives KiB
# per dispatch of a kernel; the same counters over --calibrate-copy (exactly
# 256 MiB read and 256 MiB written per dispatch) give the scale factors.  A
# summary records a hash of the kernel's sources and is used only while they
# are unchanged.
DECODE_SOURCES = ["block_quantized_kv_amd/csrc/attn_decode.hip", "block_quantized_kv_amd/csrc/kvq_device.h",
                  "block_quantized_kv_amd/csrc/kvq_layout.h", "block_quantized_kv_amd/csrc/kvq_internal.h",
                  "block_quantized_kv_amd/csrc/kvq_quant.h"]
PREFILL_SOURCES = ["block_quantized_kv_amd/csrc/attn_prefill.hip", "block_quantized_kv_amd/csrc/kvq_device.h",
                   "block_quantized_kv_amd/csrc/kvq_layout.h", "block_quantized_kv_amd/csrc/kvq_internal.h"]
TRAFFIC = {
    # which: (summary file, kernels of one launch, sources, profiled command, what one launch is)
    "decode": (os.path.join(ROOT, "profiles", "decode64k_q4g64_traffic.txt"), ["decode_kernel", "combine_kernel"],
               DECODE_SOURCES, "python -u bench.py --steps 32 --warmup 8 --step-only",
               "one decode step, kvq_append_attend_decode, 64K-context Q4_G64 decode (1 seq, 24/4 heads, "
               "head_dim 256)"),
    "prefill": (os.path.join(ROOT, "profiles", "prefill2k_over32k_traffic.txt"), ["prefill_kernel"],
                PREFILL_SOURCES, "python -u bench.py --prefill-only",
                "one kvq_attend_prefill call, 2048-token chunk over a 32768-row prefix (q8_0 K / q4_0 V, 32/8 "
                "heads, head_dim 128)"),
}


def source_hash(sources) -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _pmc_mean(path_glob: str, counter: str, name_pat: str):
    import csv
    import glob
    vals = []
    for f in glob.glob(path_glob):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter and name_pat in r["Kernel_Name"]:
                    vals.append(float(r["Counter_Value"]))
    return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)


def write_traffic_summary(which: str, pmc_dir: str):
    path, kernels, sources, cmd, what = TRAFFIC[which]
    g = lambda sub: os.path.join(pmc_dir, sub, "*_counter_collection.csv")
    fetch, write, n = {}, {}, []
    for kn in kernels:
        fetch[kn], n1 = _pmc_mean(g("fetch"), "FETCH_SIZE", kn)
        write[kn], n2 = _pmc_mean(g("write"), "WRITE_SIZE", kn)
        n.append((n1, n2))
    f_cal, _ = _pmc_mean(g("cfetch"), "FETCH_SIZE", "copy")
    w_cal, _ = _pmc_mean(g("cwrite"), "WRITE_SIZE", "copy")
    if None in list(fetch.values()) + list(write.values()) + [f_cal, w_cal]:
        sys.exit("missing counter runs under " + pmc_dir)
    kib256 = 256 * 1024  # KiB in 256 MiB
    ff, fw = kib256 / f_cal, kib256 / w_cal
    fetch_b = sum(fetch.values()) * ff * 1024
    write_b = sum(write.values()) * fw * 1024
    regex = "|".join(kernels)
    lines = [
        f"# HBM traffic of {what} ({' + '.join(kernels)}), from rocprofv3 counters",
        "#",
        "# commands (on the GPU machine, from the repo root; one counter per run):",
        f"#   rocprofv3 --pmc FETCH_SIZE --kernel-include-regex '{regex}' -d <dir>/fetch -o fetch "
        f"--output-format csv -- {cmd}",
        "#   rocprofv3 --pmc WRITE_SIZE (same, -d <dir>/write -o write)",
        "#   rocprofv3 --pmc FETCH_SIZE -d <dir>/cfetch -o cfetch --output-format csv -- python -u bench.py --calibrate-copy",
        "#   rocprofv3 --pmc WRITE_SIZE -d <dir>/cwrite -o cwrite --output-format csv -- python -u bench.py "
        "--calibrate-copy",
        f"#   python bench.py --write-traffic-summary {which} <dir>",
        f"source_hash: {source_hash(sources)}",
        f"dispatches: {' '.join(f'{a} {b}' for a, b in n)}",
    ] + [f"fetch_kib_{kn}: {fetch[kn]:.1f}" for kn in kernels] + \
        [f"write_kib_{kn}: {write[kn]:.1f}" for kn in kernels] + [
        f"copy_fetch_kib_per_256MiB: {f_cal:.1f}",
        f"copy_write_kib_per_256MiB: {w_cal:.1f}",
        f"fetch_scale: {ff:.4f}",
        f"write_scale: {fw:.4f}",
        f"traffic_bytes_per_launch: {fetch_b + write_b:.0f}",
        f"fetch_bytes_per_launch: {fetch_b:.0f}",
        f"write_bytes_per_launch: {write_b:.0f}",
    ]
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def read_traffic(which: str = "decode"):
    """Counter-backed HBM bytes per launch of a kernel, or None when the
    summary is missing or was taken on other sources."""
    path, _, sources, _, _ = TRAFFIC[which]
    try:
        kv = {}
        with open(path) as fh:
            for line in fh:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("source_hash") != source_hash(sources):
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


# ---- counter-backed matrix-core and vector activity -------------------------
# One rocprofv3 --pmc pass with the counters below over the prefill leg
# (--prefill-only) or over the decode step (--step-only).  MFMA busy fraction =
# SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x cycles), where GRBM_GUI_ACTIVE reads the
# sum of the 8 XCDs' busy cycles; SQ_INSTS_VALU includes the MFMA
# instructions; the L2 hit rate comes from TCC_HIT / TCC_MISS summed over the
# channels of every XCD.  A summary records a hash of the kernel's sources and is used
# only while they are unchanged.
BUSY_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA",
                 "SQ_INSTS_LDS", "SQ_WAVES", "GRBM_GUI_ACTIVE", "TCC_HIT_sum", "TCC_MISS_sum"]
N_SIMDS, N_XCDS = 1024, 8
BUSY_FILES = {
    "prefill": (os.path.join(ROOT, "profiles", "prefill2k_over32k_counters.txt"), "prefill_kernel", PREFILL_SOURCES,
                "python -u bench.py --prefill-only"),
    "decode": (os.path.join(ROOT, "profiles", "decode64k_q4g64_counters.txt"), "decode_kernel", DECODE_SOURCES,
               "python -u bench.py --steps 32 --warmup 8 --step-only"),
}


def write_busy_summary(which: str, pmc_dir: str):
    path, kname, sources, cmd = BUSY_FILES[which]
    g = os.path.join(pmc_dir, "*_counter_collection.csv")
    vals, n = {}, 0
    for c in BUSY_COUNTERS:
        vals[c], n = _pmc_mean(g, c, kname)
        if vals[c] is None:
            sys.exit(f"counter {c} of {kname} missing under {pmc_dir}")
    cycles = vals["GRBM_GUI_ACTIVE"] / N_XCDS
    waves = vals["SQ_WAVES"]
    lines = [
        f"# {kname}: matrix-core and vector activity per dispatch, from one rocprofv3 counter pass",
        "# command (on the GPU machine, from the repo root):",
        f"#   rocprofv3 --pmc {' '.join(BUSY_COUNTERS)} -d <dir> -o run --output-format csv -- {cmd}",
        f"#   python bench.py --write-busy-summary {which} <dir>",
        "# mfma_busy_frac = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8 XCDs)",
        "# tcc_hit_rate = TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum) (L2 requests of all 8 XCDs)",
        f"source_hash: {source_hash(sources)}",
        f"dispatches: {n}",
    ] + [f"{c}: {vals[c]:.6g}" for c in BUSY_COUNTERS] + [
        f"cycles_per_xcd: {cycles:.6g}",
        f"mfma_busy_frac: {vals['SQ_VALU_MFMA_BUSY_CYCLES'] / (N_SIMDS * cycles):.4f}",
        f"valu_insts_per_wave: {vals['SQ_INSTS_VALU'] / waves:.6g}",
        f"mfma_insts_per_wave: {vals['SQ_INSTS_MFMA'] / waves:.6g}",
        f"lds_insts_per_wave: {vals['SQ_INSTS_LDS'] / waves:.6g}",
        f"tcc_hit_rate: {vals['TCC_HIT_sum'] / max(1.0, vals['TCC_HIT_sum'] + vals['TCC_MISS_sum']):.4f}",
    ]
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def read_busy(which: str):
    """The counter summary of a kernel as a dict, or None when it is missing
    or was taken on other sources."""
    path, _, sources, _ = BUSY_FILES[which]
    try:
        kv = {}
        with open(path) as fh:
            for line in fh:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("source_hash") != source_hash(sources):
            return None
        return {"mfma_busy_frac": float(kv["mfma_busy_frac"]),
                "valu_insts_per_wave": float(kv["valu_insts_per_wave"]),
                "mfma_insts_per_wave": float(kv["mfma_insts_per_wave"]),
                "tcc_hit_rate": float(kv["tcc_hit_rate"]) if "tcc_hit_rate" in kv else None,
                "source": os.path.relpath(path, ROOT)}
    except (OSError, KeyError, ValueError):
        return None


def calibrate_copy():
    """Plain device-to-device copies of a known size: what FETCH_SIZE /
    WRITE_SIZE read for exactly 256 MiB in and 256 MiB out per dispatch."""
    import torch
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(8):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_per_dispatch": n, "dispatches": 8}))


def decode_bytes(cfg) -> dict:
    from block_quantized_kv_amd import kvq_row_code_bytes
    kc, vc = cfg.layers[0]
    d, H, n = cfg.head_dim, cfg.n_kv_heads, cfg.ctx
    row_k = kvq_row_code_bytes(kc, d) + 2 * d // (64 if kc == "q4_g64" else 32)
    row_v = kvq_row_code_bytes(vc, d) + 2 * d // (64 if vc == "q4_g64" else 32)
    kv = n * H * (row_k + row_v)
    qo = 2 * cfg.n_seqs * cfg.n_q_heads * d * 4
    app = H * d * 4 * 2 + H * (row_k + row_v)
    return {"kv": kv, "q_out": qo, "append": app, "step": kv + qo + app,
            "attend_kernel": kv + cfg.n_seqs * cfg.n_q_heads * d * 4,
            "fused_kernel": kv + cfg.n_seqs * cfg.n_q_heads * d * 4 + app}


def headline_setup(torch, dev, rotate: int, keep_host: bool = False):
    """The timed step of the headline workload, built exactly as the benchmark
    times it (the parity tests build it through this function too):
    the 64K-context Q4_G64 cache (24/4 heads, d 256) holds rows 0..65534,
    appended in 16384-row kvq_append calls; `rotate` copies of it are made
    (so timed loops can defeat the last-level cache); step(i, stream) is one
    kvq_append_attend_decode call on copy i % rotate that appends row 65535
    (k_new, v_new) and attends from the query over all 65536 rows, with the
    workspace sized by decode_workspace for that call."""
    import types

    import workloads
    from block_quantized_kv_amd import Layer, decode_workspace, kvq_append, kvq_append_attend_decode
    cfg = workloads.DECODE_64K
    kc, vc = cfg.layers[0]
    n, H, d = cfg.ctx, cfg.n_kv_heads, cfg.head_dim
    # ---- setup (untimed): fill rows 0..n-2, keep row n-1 as the step's new token
    base = Layer.create(kc, vc, d, H, 1, cfg.capacity, device=dev)
    k = workloads.kv_rows(cfg, 0, 0, "k", 0, n, dev)
    v = workloads.kv_rows(cfg, 0, 0, "v", 0, n, dev)
    for a in range(0, n - 1, 16384):
        b = min(n - 1, a + 16384)
        kvq_append(base, k[a:b].contiguous(), v[a:b].contiguous(),
                   torch.zeros(b - a, dtype=torch.int32, device=dev),
                   torch.arange(a, b, dtype=torch.int64, device=dev))
    k_new, v_new = k[n - 1:n].contiguous(), v[n - 1:n].contiguous()
    k_new2, v_new2 = k[n - 2:n].contiguous(), v[n - 2:n].contiguous()  # two drafted tokens
    host_kv = (k.cpu().numpy(), v.cpu().numpy()) if keep_host else None
    del k, v
    caches = [base] + [base.clone() for _ in range(rotate - 1)]
    q = workloads.queries(cfg, 0, dev)
    seq_len = torch.tensor([n], dtype=torch.int64, device=dev)
    ws = decode_workspace(base, cfg.n_q_heads, 1, n)
    out = torch.empty_like(q)

    def step(i, st=None):
        kvq_append_attend_decode(caches[i % rotate], k_new, v_new, q, seq_len, n, cfg.scale, out=out,
                                 workspace=ws, stream=st)

    return types.SimpleNamespace(cfg=cfg, base=base, caches=caches, k_new=k_new, v_new=v_new, k_new2=k_new2,
                                 v_new2=v_new2, host_kv=host_kv, q=q, seq_len=seq_len, ws=ws, out=out, step=step)


def main():
    args = _args()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.write_traffic_summary:
        write_traffic_summary(*args.write_traffic_summary)
        return
    if args.write_busy_summary:
        write_busy_summary(*args.write_busy_summary)
        return
    if args.prefill_only:
        import torch
        from block_quantized_kv_amd import load_library
        load_library()
        print(json.dumps(run_prefill(torch, torch.device("cuda:0"), args)), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the library has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.step_only:
        args.no_cpu_baseline = args.no_baselines = args.no_prefill = args.no_quality = True
    import workloads
    from block_quantized_kv_amd import kvq_append, kvq_attend_decode, load_library
    load_library()
    dev = torch.device("cuda:0")
    hs = headline_setup(torch, dev, ROTATE)
    cfg, base, caches, q, seq_len, ws, out = hs.cfg, hs.base, hs.caches, hs.q, hs.seq_len, hs.ws, hs.out
    k_new, v_new, k_new2, v_new2 = hs.k_new, hs.v_new, hs.k_new2, hs.v_new2
    kc, vc = cfg.layers[0]
    n, H, d = cfg.ctx, cfg.n_kv_heads, cfg.head_dim
    new_seq = torch.zeros(1, dtype=torch.int32, device=dev)
    new_pos = torch.tensor([n - 1], dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()
    step = hs.step

    def step_unfused(i, st=stream):
        L = caches[i % ROTATE]
        kvq_append(L, k_new, v_new, new_seq, new_pos, stream=st)
        kvq_attend_decode(L, q, seq_len, n, cfg.scale, out=out, workspace=ws, stream=st)

    settle(torch, step, 256)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # eager reference timing (host launches each call)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / args.steps

    # The step as captured HIP graphs: one graph holds ROTATE consecutive steps
    # (one per rotated cache; the library only enqueues kernels, so the calls
    # are capturable), plus one-step graphs for a remainder.  Serving replays
    # graphs.
    cap = torch.cuda.Stream()
    one_step, ring, unfused_ring = [], torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    attend_graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        for i in range(ROTATE):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                step(i, cap)
            one_step.append(g)
        with torch.cuda.graph(ring, stream=cap):
            for i in range(ROTATE):
                step(i, cap)
        if not args.step_only:
            with torch.cuda.graph(unfused_ring, stream=cap):
                for i in range(ROTATE):
                    step_unfused(i, cap)
            with torch.cuda.graph(attend_graph, stream=cap):
                for i in range(ROTATE):
                    kvq_attend_decode(caches[i], q, seq_len, n, cfg.scale, out=out, workspace=ws, stream=cap)
    torch.cuda.synchronize()
    settle(torch, lambda i: ring.replay(), 16)
    for _ in range(max(1, args.warmup // ROTATE)):
        ring.replay()
    torch.cuda.synchronize()

    def run_graph_steps(k):
        for _ in range(k // ROTATE):
            ring.replay()
        for i in range(k % ROTATE):
            one_step[i].replay()

    # ---- timed region: exactly `steps` steps, synchronized on both sides;
    # first as graph replays, then as eager launches (both reported; `value`
    # is the faster way of running the same steps)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_start.record()
    run_graph_steps(args.steps)
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    graph_ms = t_start.elapsed_time(t_end) / args.steps
    if eager_ms < graph_ms:
        ms_per_step, timing = eager_ms, "eager launches (stream order)"
    else:
        ms_per_step, timing = graph_ms, f"HIP-graph replay, {ROTATE} steps per graph"
    nb = decode_bytes(cfg)
    value = nb["step"] / (ms_per_step * 1e-3) / 1e9

    # ---- dominant kernel: decode_kernel, which appends and attends (with the
    # combine it is the whole step); HIP events around graphs of 16
    # back-to-back steps on the graphs' stream
    reps = max(4, args.steps // ROTATE)
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record()
    for _ in range(reps):
        ring.replay()
    a1.record()
    torch.cuda.synchronize()
    att_avg_ms = a0.elapsed_time(a1) / (reps * ROTATE)
    achieved = nb["fused_kernel"] / (att_avg_ms * 1e-3) / 1e9
    unfused_ms = attend_only_ms = None
    if not args.step_only:
        # the same step as two calls (kvq_append, kvq_attend_decode)
        u0, u1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        u0.record()
        for _ in range(reps):
            unfused_ring.replay()
        u1.record()
        torch.cuda.synchronize()
        unfused_ms = round(u0.elapsed_time(u1) / (reps * ROTATE), 5)
        # attention alone (no append)
        u0.record()
        for _ in range(reps):
            attend_graph.replay()
        u1.record()
        torch.cuda.synchronize()
        attend_only_ms = round(u0.elapsed_time(u1) / (reps * ROTATE), 5)
    traffic = read_traffic("decode")
    # the graph timing repeated 5 times (medians are steadier than one run)
    reps5 = []
    for _ in range(5):
        a0.record()
        run_graph_steps(max(ROTATE, (args.steps // 5) // ROTATE * ROTATE))
        a1.record()
        torch.cuda.synchronize()
        reps5.append(a0.elapsed_time(a1) / max(ROTATE, (args.steps // 5) // ROTATE * ROTATE))
    reps5.sort()
    speak = stream_peak(torch, dev) if not args.step_only else None

    result = {
        "metric": "decode-attention effective KV GB/s @64K ctx",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16xf16->f32 (int4 codes)",
        "data": "synthetic, seeded (N(0,1) x log-uniform per-channel scales)",
        "config": {"workload": cfg.name, "context": n, "n_q_heads": cfg.n_q_heads,
                   "n_kv_heads": H, "head_dim": d, "k_codec": kc, "v_codec": vc,
                   "step": "kvq_append_attend_decode (append 1 token + attend, one call)",
                   "rotated_caches": ROTATE,
                   "bytes_per_step": nb["step"], "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
                   # the decode target: 70 % of the HBM peak at 64K context
                   "target_pct_hbm_peak": 70.0, "meets_target": 100 * value / HBM_PEAK_GBS >= 70.0,
                   "timing": timing, "settle_ms_before_timed_loops": SETTLE_MS,
                   "eager_ms_per_step": round(eager_ms, 5),
                   "graph_ms_per_step": round(graph_ms, 5),
                   "graph_ms_per_step_median_of_5": round(reps5[2], 5),
                   "unfused_graph_ms_per_step": unfused_ms,
                   "attend_only_graph_ms": attend_only_ms,
                   "wall_s_timed_region": round(wall, 4)},
        "roofline": {"bound": "hbm",
                     "kernel": "kvq_append_attend_decode = decode_kernel<256,Q4_G64,Q4_G64> (append + attention)"
                               " + combine_kernel<256>",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "bytes_per_launch": nb["fused_kernel"], "avg_launch_ms": round(att_avg_ms, 5),
                     "stream_read_peak_gbs": speak["gbs"] if speak else None,
                     "frac_of_stream_read_peak": round(achieved / speak["gbs"], 4) if speak else None,
                     "counters": read_busy("decode")},
    }

    if not args.step_only:
        run_multi_query(torch, dev, cfg, caches, k_new2, v_new2, seq_len, nb, args, stream, result)
        result["paged"] = run_paged(torch, dev, cfg, base, k_new, v_new, q, seq_len, nb, args)
        result["long_context"] = run_long_context(torch, dev, args)
        result["decode_32k"] = run_decode_config(torch, dev, args, workloads.DECODE_32K, rotate=20)
        result["batched_decode"] = run_decode_config(torch, dev, args, workloads.BATCHED, rotate=1)
    if speak is not None:
        result["stream_read_peak"] = speak
    if not args.no_baselines:
        result["f16_control"] = run_f16_control(torch, dev, args)
    if not args.no_prefill:
        result["prefill"] = run_prefill(torch, dev, args)
        if result["prefill"].get("status") != "unavailable":
            result["prefill"]["other_head_dims"] = run_prefill_other_dims(torch, dev)
    if not args.no_quality:
        result["quality"] = run_quality(torch, dev, args)

    if not args.no_cpu_baseline:
        cb = cpu_baselines(torch, dev)
        per = cb["per_config"]
        h = per[cfg.name]
        result["cpu_baseline"] = {
            "value": h["value"], "unit": "GB/s", "cores": cb["threads"], "kind": "oracle",
            "sample": f"the whole 64K-context step (dequantize all 65536 rows of the 4 kv-heads, binary64 "
                      f"attention of all 24 q-heads) on {cb['threads']} threads, {h['seconds']} s",
            "single_thread": h.get("single_thread"), "cpu_model": cb["cpu_model"], "nproc": cb["nproc"],
            "per_config": per}
        # the oracle beside each GPU figure
        for leg, name in (("decode_32k", workloads.DECODE_32K.name), ("long_context", workloads.DECODE_196K.name),
                          ("batched_decode", workloads.BATCHED.name)):
            if leg in result:
                result[leg]["cpu_oracle"] = per[name]
        if "prefill" in result:
            result["prefill"]["cpu_oracle"] = per["prefill_2048_over_32768"]
    print(json.dumps(result), flush=True)


def stream_peak(torch, dev, reps: int = 48) -> dict:
    """Measured streaming-read rate of this GPU: kvq_probe_stream_read over 64 MiB windows
    rotating through 1 GiB (so the 256 MB last-level cache cannot serve them),
    for 256, 512 and 1024 workgroups of 8 waves; the best is the practical
    ceiling the decode roofline is also quoted against."""
    from block_quantized_kv_amd.probe import kvq_probe_stream_read
    win, total = 64 << 20, 1 << 30
    buf = torch.ones(total, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    by = {}
    for nwg in (256, 512, 1024):
        settle(torch, lambda i: kvq_probe_stream_read(buf[(i % 4) * win:(i % 4 + 1) * win], nwg, sink), 16, 100.0)
        e0.record()
        for i in range(reps):
            j = i % (total // win)
            kvq_probe_stream_read(buf[j * win:(j + 1) * win], nwg, sink)
        e1.record()
        torch.cuda.synchronize()
        by[str(nwg)] = round(win * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del buf
    return {"gbs": max(by.values()), "by_workgroups_of_8_waves": by, "bytes_per_launch": win}


def run_long_context(torch, dev, args) -> dict:
    """The 196K-context split-KV configuration: four layers (layer 0 q8_0 K/V,
    layers 1-3 Q4_G64), one kvq_attend_decode per layer per step, timed as
    HIP-graph replays of the four calls (1.07 GB of K/V per step, so no
    rotation is needed)."""
    import workloads
    from block_quantized_kv_amd import Layer, decode_workspace, kvq_append, kvq_attend_decode
    cfg = workloads.DECODE_196K
    n, H, d = cfg.ctx, cfg.n_kv_heads, cfg.head_dim
    layers, qs, outs, kv_bytes = [], [], [], []
    for li, (kc, vc) in enumerate(cfg.layers):
        L = Layer.create(kc, vc, d, H, 1, cfg.capacity, device=dev)
        for a in range(0, n, 32768):
            b = min(n, a + 32768)
            k = workloads.kv_rows(cfg, li, 0, "k", a, b - a, dev)
            v = workloads.kv_rows(cfg, li, 0, "v", a, b - a, dev)
            kvq_append(L, k, v, torch.zeros(b - a, dtype=torch.int32, device=dev),
                       torch.arange(a, b, dtype=torch.int64, device=dev))
            del k, v
        layers.append(L)
        qs.append(workloads.queries(cfg, li, dev))
        outs.append(torch.empty_like(qs[-1]))
        kv_bytes.append(L.k.nbytes + L.v.nbytes)
    ws = decode_workspace(layers[0], cfg.n_q_heads, 1, n)
    lens = torch.tensor([n], dtype=torch.int64, device=dev)
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        for li, L in enumerate(layers):
            kvq_attend_decode(L, qs[li], lens, n, cfg.scale, out=outs[li], workspace=ws, stream=cap)
        with torch.cuda.graph(g, stream=cap):
            for li, L in enumerate(layers):
                kvq_attend_decode(L, qs[li], lens, n, cfg.scale, out=outs[li], workspace=ws, stream=cap)
    torch.cuda.synchronize()
    reps = max(8, args.steps // 16)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    settle(torch, lambda i: g.replay(), 4)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    total = sum(kv_bytes)
    del layers
    return {"workload": cfg.name, "context": n, "layers": [f"{kc}/{vc}" for kc, vc in cfg.layers],
            "ms_per_step": round(ms, 5), "kv_bytes_per_step": total,
            "value": round(total / (ms * 1e-3) / 1e9, 2), "unit": "GB/s",
            "step": "4 x kvq_attend_decode (one per layer), HIP-graph replay"}


def run_decode_config(torch, dev, args, cfg, rotate: int) -> dict:
    """Attention-only decode of a workload configuration over all of its
    sequences: one kvq_attend_decode call per step, timed as HIP-graph replays
    that rotate over `rotate` independent caches (so the 256 MB MALL cannot
    serve a call's K/V).  Algorithmic bytes: the quantized K and V of every
    attended row, once per kv-head."""
    import workloads
    from block_quantized_kv_amd import Layer, decode_workspace, kvq_append, kvq_attend_decode
    (kc, vc), = cfg.layers
    H, d = cfg.n_kv_heads, cfg.head_dim
    lens = workloads.seq_lengths(cfg, dev)
    lens_h = [int(x) for x in lens.cpu()]
    base = Layer.create(kc, vc, d, H, cfg.n_seqs, cfg.capacity, device=dev)
    for b, n in enumerate(lens_h):
        for a in range(0, n, 32768):
            e = min(n, a + 32768)
            k = workloads.kv_rows(cfg, 0, b, "k", a, e - a, dev)
            v = workloads.kv_rows(cfg, 0, b, "v", a, e - a, dev)
            kvq_append(base, k, v, torch.full((e - a,), b, dtype=torch.int32, device=dev),
                       torch.arange(a, e, dtype=torch.int64, device=dev))
            del k, v
    caches = [base] + [base.clone() for _ in range(rotate - 1)]
    q = workloads.queries(cfg, 0, dev)
    out = torch.empty_like(q)
    max_len = max(lens_h)
    ws = decode_workspace(base, cfg.n_q_heads, cfg.n_seqs, max_len)
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    per_graph = max(4, rotate)
    with torch.cuda.stream(cap):
        for i in range(per_graph):
            kvq_attend_decode(caches[i % rotate], q, lens, max_len, cfg.scale, out=out, workspace=ws, stream=cap)
        with torch.cuda.graph(g, stream=cap):
            for i in range(per_graph):
                kvq_attend_decode(caches[i % rotate], q, lens, max_len, cfg.scale, out=out, workspace=ws,
                                  stream=cap)
    torch.cuda.synchronize()
    reps = max(4, args.steps // (4 * per_graph))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    settle(torch, lambda i: g.replay(), 4)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (reps * per_graph)
    row_bytes = sum(r + 2 * (d // (64 if c == "q4_g64" else 32))
                    for r, c in ((d if kc == "q8_0" else d // 2, kc), (d if vc == "q8_0" else d // 2, vc)))
    kv = sum(lens_h) * H * row_bytes
    del caches, base
    gbs = kv / (ms * 1e-3) / 1e9
    return {"workload": cfg.name, "n_seqs": cfg.n_seqs, "lengths": lens_h if cfg.n_seqs > 1 else lens_h[0],
            "n_q_heads": cfg.n_q_heads, "n_kv_heads": H, "head_dim": d, "k_codec": kc, "v_codec": vc,
            "ms_per_call": round(ms, 5), "kv_bytes_per_call": kv, "rotated_caches": rotate,
            "value": round(gbs, 2), "unit": "GB/s", "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "step": "kvq_attend_decode over every sequence, HIP-graph replay"}


def run_paged(torch, dev, cfg, base, k_new, v_new, q, seq_len, nb, args) -> dict:
    """The same step over paged planes: each rotated cache is a pool of
    256-row pages in shuffled order, reached through a block table."""
    import numpy as np
    from block_quantized_kv_amd import Layer, PagedLayer, kvq_paged_append_attend_decode_mq, paged_decode_workspace
    n, d, H = cfg.ctx, cfg.head_dim, cfg.n_kv_heads
    R, npg = 256, cfg.ctx // 256
    pools = []
    for r in range(ROTATE):
        perm = np.random.default_rng(100 + r).permutation(npg).astype(np.int32)
        pool = Layer.create(base.k.codec, base.v.codec, d, H, npg, R, device=dev, zero=False)
        # page perm[i] holds rows [i*R, (i+1)*R) of the contiguous cache
        for src, dst in ((base.k, pool.k), (base.v, pool.v)):
            for t_src, t_dst in ((src.codes, dst.codes), (src.scales, dst.scales)):
                per = t_src.numel() // (H * npg)
                view_src = t_src.view(H, npg, per)
                view_dst = t_dst.view(npg, H, per)
                view_dst[torch.from_numpy(perm).to(dev).long()] = view_src.transpose(0, 1)
        pools.append(PagedLayer(pool, torch.from_numpy(perm[None]).to(dev)))
    kn, vn, q1 = k_new[None].contiguous(), v_new[None].contiguous(), q[:, None].contiguous()
    out = torch.empty_like(q1)
    ws = paged_decode_workspace(pools[0], cfg.n_q_heads, 1, 1, n)
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        for i in range(ROTATE):  # warm the kernels before capture
            kvq_paged_append_attend_decode_mq(pools[i], kn, vn, q1, seq_len, n, cfg.scale, out=out, workspace=ws,
                                              stream=cap)
        with torch.cuda.graph(g, stream=cap):
            for i in range(ROTATE):
                kvq_paged_append_attend_decode_mq(pools[i], kn, vn, q1, seq_len, n, cfg.scale, out=out,
                                                  workspace=ws, stream=cap)
    torch.cuda.synchronize()
    reps = max(4, args.steps // ROTATE)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    settle(torch, lambda i: g.replay(), 16)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (reps * ROTATE)
    del pools
    return {"ms_per_step": round(ms, 5), "value": round(nb["step"] / (ms * 1e-3) / 1e9, 2), "unit": "GB/s",
            "page_rows": R, "pages": npg, "order": "shuffled",
            "step": "kvq_paged_append_attend_decode_mq (q_len 1), HIP-graph replay"}


def run_multi_query(torch, dev, cfg, caches, k_new2, v_new2, seq_len, nb, args, stream, result):
    # ---- the same step verifying two drafted tokens (multi-query decode):
    # append rows n-2 and n-1, attend from both; the K/V bytes are read once
    from block_quantized_kv_amd import decode_mq_workspace, kvq_append_attend_decode_mq
    n, d = cfg.ctx, cfg.head_dim
    q2 = torch.randn(1, 2, cfg.n_q_heads, d, device=dev, generator=torch.Generator(device=dev).manual_seed(2))
    out2 = torch.empty_like(q2)
    ws2 = decode_mq_workspace(caches[0], cfg.n_q_heads, 1, 2, n)
    k_new2, v_new2 = k_new2[None], v_new2[None]  # [n_seqs][q_len][H][d]

    def step2(i):
        kvq_append_attend_decode_mq(caches[i % ROTATE], k_new2, v_new2, q2, seq_len, n, cfg.scale, out=out2,
                                    workspace=ws2, stream=stream)

    settle(torch, step2, 256)
    for i in range(args.warmup):
        step2(i)
    torch.cuda.synchronize()
    m0, m1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    m0.record(stream)
    for i in range(args.steps):
        step2(i)
    m1.record(stream)
    torch.cuda.synchronize()
    mq_ms = m0.elapsed_time(m1) / args.steps
    mq_bytes = nb["kv"] + 2 * nb["q_out"] + 2 * nb["append"]
    result["multi_query"] = {"q_len": 2, "ms_per_step": round(mq_ms, 5),
                             "value": round(mq_bytes / (mq_ms * 1e-3) / 1e9, 2), "unit": "GB/s",
                             "tokens_per_s": round(2 / (mq_ms * 1e-3), 1),
                             "step": "kvq_append_attend_decode_mq (append 2 tokens + attend from both), eager"}


def run_prefill(torch, dev, args):
    """2048-token causal chunk over a 32768-token quantized prefix (q8_0 K / q4_0 V)."""
    import workloads
    from block_quantized_kv_amd import Layer, kvq_append, kvq_attend_prefill
    from block_quantized_kv_amd._binding import KvqError
    P, T = workloads.PREFILL["prefix"], workloads.PREFILL["chunk"]
    hq, hkv, d = workloads.PREFILL["n_q_heads"], workloads.PREFILL["n_kv_heads"], workloads.PREFILL["head_dim"]
    kc, vc = workloads.PREFILL["k_codec"], workloads.PREFILL["v_codec"]
    layer = Layer.create(kc, vc, d, hkv, 1, P + T, device=dev)
    q, k, v = workloads.prefill_inputs(dev)
    for a in range(0, P + T, 16384):
        b = min(P + T, a + 16384)
        kvq_append(layer, k[a:b].contiguous(), v[a:b].contiguous(),
                   torch.zeros(b - a, dtype=torch.int32, device=dev),
                   torch.arange(a, b, dtype=torch.int64, device=dev))
    flops = 4.0 * d * hq * sum(P + t + 1 for t in range(T))
    try:
        kvq_attend_prefill(layer, q, 0, P, 1.0 / d ** 0.5)
    except KvqError as e:
        return {"status": "unavailable", "reason": str(e)}
    # the chunk's own append (quantize-on-write of its 2048 rows x kv-heads),
    # which precedes the attention in a prefill step; it rewrites the same
    # rows with the same values, so the cache is unchanged
    kc_chunk, vc_chunk = k[P:P + T].contiguous(), v[P:P + T].contiguous()
    seq0 = torch.zeros(T, dtype=torch.int32, device=dev)
    pos = torch.arange(P, P + T, dtype=torch.int64, device=dev)
    for _ in range(3):
        kvq_append(layer, kc_chunk, vc_chunk, seq0, pos)
    torch.cuda.synchronize()
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record()
    for _ in range(20):
        kvq_append(layer, kc_chunk, vc_chunk, seq0, pos)
    a1.record()
    torch.cuda.synchronize()
    append_ms = a0.elapsed_time(a1) / 20
    append_in = 2 * T * hkv * d * 4
    append_out = T * hkv * sum(r + 2 * (d // (64 if c == "q4_g64" else 32))
                               for r, c in ((d if kc == "q8_0" else d // 2, kc), (d if vc == "q8_0" else d // 2, vc)))
    out = torch.empty(T, hq, d, device=dev)
    settle(torch, lambda i: kvq_attend_prefill(layer, q, 0, P, 1.0 / d ** 0.5, out=out), 8)
    reps = 20
    a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a_ev.record()
    for _ in range(reps):
        kvq_attend_prefill(layer, q, 0, P, 1.0 / d ** 0.5, out=out)
    b_ev.record()
    torch.cuda.synchronize()
    ms = a_ev.elapsed_time(b_ev) / reps
    tf = flops / (ms * 1e-3) / 1e12
    mp = mfma_peak(torch, dev)
    kv_bytes = (P + T) * hkv * sum(r + 2 * (d // (64 if c == "q4_g64" else 32))
                                   for r, c in ((d if kc == "q8_0" else d // 2, kc), (d if vc == "q8_0" else d // 2, vc)))
    return {"metric": "prefill TFLOP/s", "value": round(tf, 2), "unit": "TFLOP/s",
            "ms_per_chunk": round(ms, 4), "flop": flops,
            "chunk_append": {"ms": round(append_ms, 4), "bytes_in": append_in, "bytes_out": append_out,
                             "gbs": round((append_in + append_out) / (append_ms * 1e-3) / 1e9, 1),
                             "step": "kvq_append of the chunk's 2048 rows (K and V, all kv-heads)"},
            "config": {"prefix": P, "chunk": T, "n_q_heads": hq, "n_kv_heads": hkv, "head_dim": d,
                       "k_codec": kc, "v_codec": vc, "timed_calls": reps, "settle_ms_before_timed_loop": SETTLE_MS},
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                         "traffic": read_traffic("prefill"), "kv_bytes": kv_bytes,
                         "measured_mfma_peak": mp, "frac_of_measured_mfma_peak": round(tf / mp["tflops"], 4),
                         "counters": read_busy("prefill")}}


def run_prefill_other_dims(torch, dev) -> list:
    """The same 2048-token chunk over a 32768-row prefix at the other head
    dims the kernel builds: 256 with the 64K decode model's heads (24/4, Q4_G64
    and q8_0/q4_0) and 64 (32/8, q8_0/q4_0); 20 timed calls after a settling
    run of the same call each.  Context for the head_dim 128 figure above, not a separate
    workload."""
    import workloads
    from block_quantized_kv_amd import Layer, kvq_append, kvq_attend_prefill
    P, T = workloads.PREFILL["prefix"], workloads.PREFILL["chunk"]
    res = []
    for d, hq, hkv, kc, vc in ((256, 24, 4, "q4_g64", "q4_g64"), (256, 24, 4, "q8_0", "q4_0"),
                               (64, 32, 8, "q8_0", "q4_0")):
        q, k, v = workloads.prefill_inputs(dev, prefix=P, chunk=T, n_q_heads=hq, n_kv_heads=hkv, head_dim=d)
        layer = Layer.create(kc, vc, d, hkv, 1, P + T, device=dev)
        for a in range(0, P + T, 16384):
            b = min(P + T, a + 16384)
            kvq_append(layer, k[a:b].contiguous(), v[a:b].contiguous(),
                       torch.zeros(b - a, dtype=torch.int32, device=dev),
                       torch.arange(a, b, dtype=torch.int64, device=dev))
        out = torch.empty(T, hq, d, device=dev)
        settle(torch, lambda i: kvq_attend_prefill(layer, q, 0, P, 1.0 / d ** 0.5, out=out), 8)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            kvq_attend_prefill(layer, q, 0, P, 1.0 / d ** 0.5, out=out)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 20
        tf = 4.0 * d * hq * sum(P + t + 1 for t in range(T)) / (ms * 1e-3) / 1e12
        res.append({"head_dim": d, "n_q_heads": hq, "n_kv_heads": hkv, "k_codec": kc, "v_codec": vc,
                    "ms_per_chunk": round(ms, 4), "tflops": round(tf, 2),
                    "frac_of_peak": round(tf / BF16_PEAK_TFLOPS, 4)})
        del layer, q, k, v, out
    return res


def mfma_peak(torch, dev) -> dict:
    """Measured matrix-core peak of this GPU: kvq_probe_mfma_f16 (a register-only loop of
    v_mfma_f32_16x16x32_f16, the prefill kernel's product) for 256, 512 and
    1024 workgroups of 8 waves; the best is the practical ceiling the prefill
    roofline is also quoted against."""
    from block_quantized_kv_amd.probe import kvq_probe_mfma_f16
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    by = {}
    for nwg in (256, 512, 1024):
        iters = 4096 * 256 // nwg
        settle(torch, lambda i: kvq_probe_mfma_f16(nwg, iters, sink), 8, 100.0)
        flop = 0.0
        e0.record()
        for _ in range(5):
            flop += kvq_probe_mfma_f16(nwg, iters, sink)
        e1.record()
        torch.cuda.synchronize()
        by[str(nwg)] = round(flop / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
    return {"tflops": max(by.values()), "by_workgroups_of_8_waves": by, "instruction": "v_mfma_f32_16x16x32_f16"}


def _time_attend(torch, caches, q, lens, max_len, scale, reps: int) -> float:
    """ms per kvq_attend_decode call, as HIP-graph replays of one call per
    cache in turn (the caches rotate so the last-level cache cannot serve
    the K/V)."""
    from block_quantized_kv_amd import decode_workspace, kvq_attend_decode
    out = torch.empty_like(q)
    ws = decode_workspace(caches[0], q.shape[1], q.shape[0], max_len)
    per_graph = max(4, len(caches))
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        for i in range(per_graph):
            kvq_attend_decode(caches[i % len(caches)], q, lens, max_len, scale, out=out, workspace=ws, stream=cap)
        with torch.cuda.graph(g, stream=cap):
            for i in range(per_graph):
                kvq_attend_decode(caches[i % len(caches)], q, lens, max_len, scale, out=out, workspace=ws,
                                  stream=cap)
    torch.cuda.synchronize()
    settle(torch, lambda i: g.replay(), 4)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * per_graph)


def run_f16_control(torch, dev, args) -> dict:
    """The pages' comparison through this library's own decode kernel: a
    q8_0 K / q4_0 V cache read directly against the f16 K / f16 V control
    (the fallback the quantized pair replaced), same kernel, same rows (the
    32K workload's outlier-channel rows), 32/8 heads, head_dim 128, at 32K
    and 65K context.  Beside it, the HBM bytes any dequant-once step moves
    (read the quantized cache, write a binary16 copy, read the copy) and the
    time they take at the 8 TB/s peak."""
    import dataclasses

    import workloads
    from block_quantized_kv_amd import Layer, kvq_append
    base = workloads.DECODE_32K
    res = {}
    for ctx in (32768, 65536):
        cfg = dataclasses.replace(base, ctx=ctx, name=f"decode_ctx{ctx // 1024}k_32q_8kv_d128")
        q = workloads.queries(cfg, 0, dev)
        lens = torch.tensor([ctx], dtype=torch.int64, device=dev)
        entry = {}
        for kc, vc in (("q8_0", "q4_0"), ("f16", "f16")):
            L = Layer.create(kc, vc, cfg.head_dim, cfg.n_kv_heads, 1, ctx, device=dev)
            for a in range(0, ctx, 16384):
                b = min(ctx, a + 16384)
                kvq_append(L, workloads.kv_rows(cfg, 0, 0, "k", a, b - a, dev),
                           workloads.kv_rows(cfg, 0, 0, "v", a, b - a, dev),
                           torch.zeros(b - a, dtype=torch.int32, device=dev),
                           torch.arange(a, b, dtype=torch.int64, device=dev))
            rot = max(2, -(-(1 << 30) // L.nbytes))
            caches = [L] + [L.clone() for _ in range(rot - 1)]
            ms = _time_attend(torch, caches, q, lens, ctx, cfg.scale, max(4, args.steps // 40))
            entry[f"{kc}/{vc}"] = {"us_per_call": round(ms * 1e3, 2), "kv_bytes": L.nbytes,
                                   "gbs": round(L.nbytes / (ms * 1e-3) / 1e9, 1), "rotated_caches": rot}
            if kc == "q8_0":
                quant_bytes = L.nbytes
            del caches, L
        f16_bytes = entry["f16/f16"]["kv_bytes"]
        entry["speedup_q8_0_q4_0_over_f16"] = round(entry["f16/f16"]["us_per_call"] /
                                                    entry["q8_0/q4_0"]["us_per_call"], 3)
        floor = quant_bytes + 2 * f16_bytes
        entry["dequant_once_hbm_floor"] = {"bytes": floor, "us_at_8tbs": round(floor / (HBM_PEAK_GBS * 1e9) * 1e6, 2)}
        res[cfg.name] = entry
    res["step"] = "kvq_attend_decode over the whole cache, HIP-graph replay, both caches through the same kernel"
    return res


def run_quality(torch, dev, args):
    """Model-free quality of the codecs (the pages' KL-divergence runs need the
    model): on the 32K (outlier channels) and 64K (per-channel scales)
    decode distributions, the GPU decode output over each codec pair against
    exact binary64 attention over the unquantized fp32 K/V, and the softmax KL
    divergence between attention over the exact keys and over the keys as the
    GPU dequantizes them (mean and max over query heads, nats)."""
    import workloads
    from block_quantized_kv_amd import Layer, kvq_append, kvq_attend_decode, kvq_dequant
    res = {}
    for cfg in (workloads.DECODE_32K, workloads.DECODE_64K):
        n, H, d, hq = cfg.ctx, cfg.n_kv_heads, cfg.head_dim, cfg.n_q_heads
        G = hq // H
        k = workloads.kv_rows(cfg, 0, 0, "k", 0, n, dev)
        v = workloads.kv_rows(cfg, 0, 0, "v", 0, n, dev)
        q = workloads.queries(cfg, 0, dev)
        kd = k.double().cpu().permute(1, 0, 2)      # [H][n][d]
        vd = v.double().cpu().permute(1, 0, 2)
        qd = q[0].double().cpu().view(H, G, d)
        s_exact = torch.einsum("hgd,hnd->hgn", qd, kd) * cfg.scale
        p_exact = torch.softmax(s_exact, dim=-1)
        ref = torch.einsum("hgn,hnd->hgd", p_exact, vd).reshape(hq, d)
        logp_exact = torch.log_softmax(s_exact, dim=-1)
        entry = {}
        for kc, vc in (("q8_0", "q8_0"), ("q4_0", "q4_0"), ("q4_g64", "q4_g64"), ("q8_0", "q4_0")):
            layer = Layer.create(kc, vc, d, H, 1, cfg.capacity, device=dev)
            for a in range(0, n, 16384):
                b = min(n, a + 16384)
                kvq_append(layer, k[a:b].contiguous(), v[a:b].contiguous(),
                           torch.zeros(b - a, dtype=torch.int32, device=dev),
                           torch.arange(a, b, dtype=torch.int64, device=dev))
            out = kvq_attend_decode(layer, q, torch.tensor([n], dtype=torch.int64, device=dev), n,
                                    cfg.scale)[0].double().cpu()
            khat = kvq_dequant(layer.k, 0, 0, n).double().cpu()
            s_q = torch.einsum("hgd,hnd->hgn", qd, khat) * cfg.scale
            kl = (p_exact * (logp_exact - torch.log_softmax(s_q, dim=-1))).sum(-1).reshape(-1)
            err = (out - ref).abs()
            entry[f"{kc}/{vc}"] = {
                "out_max_rel_err": round(float(err.max() / ref.abs().max()), 6),
                "out_rms_rel_err": round(float(err.pow(2).sum().sqrt() / ref.pow(2).sum().sqrt()), 6),
                "softmax_kl_mean": float(f"{kl.mean().item():.4e}"),
                "softmax_kl_max": float(f"{kl.max().item():.4e}")}
            del layer
        res[cfg.name] = entry
    return res


# ---- the CPU oracle beside every result ------------------------------------
# The oracle is plain single-threaded C (oracle/kvq_oracle.c); its decode step
# is "dequantize the cached rows, then binary64 attention".  Here it runs on
# the host's cores with one task per (sequence, kv-head) dequantization and
# one per (sequence, q-head) attention (ctypes releases the interpreter lock
# during each call), and, for the three smallest configurations, on one
# thread as well.  Quantizing the rows into the oracle's own codes is setup,
# as filling the cache is for the GPU.

CPU_THREADS_MAX = 16  # the host share of one GPU


def cpu_info() -> dict:
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(),
            "threads": max(1, min(CPU_THREADS_MAX, os.cpu_count() or 1))}


def _oracle_codes(pool, codec, rows_nhd):
    """rows fp32 [n][H][d] -> [(codes, scales)] per kv-head (setup, threaded)."""
    import numpy as np

    import oracle
    H = rows_nhd.shape[1]
    return list(pool.map(lambda g: oracle.quantize_rows(codec, np.ascontiguousarray(rows_nhd[:, g])), range(H)))


def _oracle_decode_seq(pool, kc, vc, d, kcodes, vcodes, q_hd, n, scale):
    """One sequence's oracle decode step: dequantize every kv-head's K and V
    rows, then attend from every q-head (each a task of `pool`)."""
    import oracle
    H = len(kcodes)
    G = q_hd.shape[0] // H
    hats = list(pool.map(lambda g: (oracle.dequant_rows(kc, kcodes[g][0], kcodes[g][1], d)[None],
                                    oracle.dequant_rows(vc, vcodes[g][0], vcodes[g][1], d)[None]), range(H)))
    list(pool.map(lambda h: oracle.attend_decode(q_hd[h:h + 1], hats[h // G][0], hats[h // G][1], n, scale),
                  range(q_hd.shape[0])))


def cpu_decode_config(torch, dev, cfg, layers, threads, single_thread: bool) -> dict:
    """The oracle's decode step of a whole configuration (every sequence, every
    q-head of the given layers) on `threads` threads, and on one thread if
    asked; value in GB/s of the same algorithmic bytes as the GPU figure."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    import workloads
    oracle._load()
    d, H = cfg.head_dim, cfg.n_kv_heads
    lens = [int(x) for x in workloads.seq_lengths(cfg, "cpu")]
    kv_bytes = 0
    t_mt = t_st = 0.0
    with ThreadPoolExecutor(threads) as pool, ThreadPoolExecutor(1) as one:
        for li in layers:
            kc, vc = cfg.layers[li]
            row = sum(r + 2 * (d // (64 if c == "q4_g64" else 32))
                      for r, c in ((d if kc == "q8_0" else d // 2, kc), (d if vc == "q8_0" else d // 2, vc)))
            q = workloads.queries(cfg, li, dev).cpu().numpy()
            for b, n in enumerate(lens):
                k = workloads.kv_rows(cfg, li, b, "k", 0, n, dev).cpu().numpy()
                v = workloads.kv_rows(cfg, li, b, "v", 0, n, dev).cpu().numpy()
                kcodes, vcodes = _oracle_codes(pool, kc, k), _oracle_codes(pool, vc, v)
                del k, v
                t0 = time.perf_counter()
                _oracle_decode_seq(pool, kc, vc, d, kcodes, vcodes, q[b], n, cfg.scale)
                t_mt += time.perf_counter() - t0
                if single_thread:
                    t0 = time.perf_counter()
                    _oracle_decode_seq(one, kc, vc, d, kcodes, vcodes, q[b], n, cfg.scale)
                    t_st += time.perf_counter() - t0
                kv_bytes += n * H * row
    r = {"value": round(kv_bytes / t_mt / 1e9, 4), "unit": "GB/s", "threads": threads, "seconds": round(t_mt, 3),
         "kv_bytes": kv_bytes,
         "sample": f"whole step: {len(lens)} sequence(s) x {cfg.n_q_heads} q-heads x {len(layers)} layer(s)"}
    if single_thread:
        r["single_thread"] = {"value": round(kv_bytes / t_st / 1e9, 4), "unit": "GB/s", "seconds": round(t_st, 3)}
    return r


def cpu_prefill(torch, dev, threads, n_rows: int = 1024) -> dict:
    """The oracle's chunked prefill (2048 tokens over a 32768-row prefix, q8_0 K /
    q4_0 V, 32/8 heads, d 128) on a sample of n_rows (token, head) rows spread
    evenly over the chunk and the heads; value in GFLOP/s of the causal flop
    count (4 d per (row, attended row)) of the sample."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    import workloads
    oracle._load()
    W = workloads.PREFILL
    P, T, hq, H, d = W["prefix"], W["chunk"], W["n_q_heads"], W["n_kv_heads"], W["head_dim"]
    kc, vc = W["k_codec"], W["v_codec"]
    q, k, v = workloads.prefill_inputs(dev)
    qn, k, v = q.float().cpu().numpy(), k.cpu().numpy(), v.cpu().numpy()
    idx = np.linspace(0, T * hq - 1, n_rows).astype(np.int64)
    toks, heads = (idx // hq).astype(np.int32), (idx % hq).astype(np.int32)
    flop = float(sum(4 * d * (P + int(t) + 1) for t in toks))
    with ThreadPoolExecutor(threads) as pool:
        kcodes, vcodes = _oracle_codes(pool, kc, k), _oracle_codes(pool, vc, v)
        del k, v
        t0 = time.perf_counter()
        hats = list(pool.map(lambda g: (oracle.dequant_rows(kc, kcodes[g][0], kcodes[g][1], d),
                                        oracle.dequant_rows(vc, vcodes[g][0], vcodes[g][1], d)), range(H)))
        kh = np.stack([x[0] for x in hats])
        vh = np.stack([x[1] for x in hats])
        pieces = np.array_split(np.arange(n_rows), 4 * threads)
        list(pool.map(lambda ix: oracle.attend_prefill(qn, kh, vh, P, 1.0 / np.sqrt(d), tokens=toks[ix],
                                                       heads=heads[ix]), pieces))
        el = time.perf_counter() - t0
    return {"value": round(flop / el / 1e9, 3), "unit": "GFLOP/s", "threads": threads, "seconds": round(el, 3),
            "flop": flop, "sample": f"{n_rows} of the {T * hq} (token, head) rows, evenly spaced"}


def cpu_baselines(torch, dev) -> dict:
    """The oracle beside every configuration (see the section comment)."""
    import workloads
    info = cpu_info()
    th = info["threads"]
    per = {}
    for cfg, layers, st in ((workloads.TINY, [0], True), (workloads.DECODE_32K, [0], True),
                            (workloads.DECODE_64K, [0], True), (workloads.DECODE_196K, [0, 1, 2, 3], False),
                            (workloads.BATCHED, [0], False)):
        per[cfg.name] = cpu_decode_config(torch, dev, cfg, layers, th, st)
    per["prefill_2048_over_32768"] = cpu_prefill(torch, dev, th)
    return dict(info, per_config=per)


if __name__ == "__main__":
    main()
