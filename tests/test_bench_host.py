"""Host logic of bench.py, no GPU: the algorithmic byte counts of the 64K
step, the counter summaries (written from rocprofv3-style CSVs and read back
only while the kernel sources are unchanged) and the one-GPU rule."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import workloads  # noqa: E402

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for i, (kernel, counter, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": value})


def test_step_bytes_of_the_64k_workload():
    # 65536 rows x 4 kv-heads x (136 + 136) B of Q4_G64 K and V at head_dim 256
    # (128 code bytes + 4 binary16 scales per row and plane)
    nb = bench.decode_bytes(workloads.DECODE_64K)
    assert nb["kv"] == 71_303_168
    assert nb["q_out"] == 2 * 24 * 256 * 4
    assert nb["append"] == 4 * 256 * 4 * 2 + 4 * 272
    assert nb["step"] == 71_361_600


def test_traffic_summary_round_trip(tmp_path, monkeypatch):
    d = tmp_path / "pmc"
    # two dispatches each; the copy calibration reads 2x and writes 1x its
    # 256 MiB (in KiB), as the counters do on the machine
    _csv(str(d / "fetch" / "f_counter_collection.csv"),
         [("decode_kernel<256>", "FETCH_SIZE", 1000.0), ("decode_kernel<256>", "FETCH_SIZE", 1200.0),
          ("combine_kernel<256>", "FETCH_SIZE", 50.0)])
    _csv(str(d / "write" / "w_counter_collection.csv"),
         [("decode_kernel<256>", "WRITE_SIZE", 80.0), ("combine_kernel<256>", "WRITE_SIZE", 4.0)])
    _csv(str(d / "cfetch" / "c_counter_collection.csv"), [("copyBuffer", "FETCH_SIZE", 131072.0)])
    _csv(str(d / "cwrite" / "c_counter_collection.csv"), [("copyBuffer", "WRITE_SIZE", 262144.0)])
    out = tmp_path / "traffic.txt"
    path, kernels, sources, cmd, what = bench.TRAFFIC["decode"]
    monkeypatch.setitem(bench.TRAFFIC, "decode", (str(out), kernels, sources, cmd, what))
    bench.write_traffic_summary("decode", str(d))
    fetch = (1100.0 + 50.0) * 2.0 * 1024
    write = (80.0 + 4.0) * 1.0 * 1024
    assert bench.read_traffic("decode") == pytest.approx(fetch + write, rel=1e-6)
    # a summary taken on other sources is not used
    text = out.read_text().replace(bench.source_hash(sources), "0000000000000000")
    out.write_text(text)
    assert bench.read_traffic("decode") is None


def test_prefill_traffic_summary(tmp_path, monkeypatch):
    d = tmp_path / "pmc"
    _csv(str(d / "fetch" / "f_counter_collection.csv"), [("prefill_kernel<128>", "FETCH_SIZE", 60000.0)])
    _csv(str(d / "write" / "w_counter_collection.csv"), [("prefill_kernel<128>", "WRITE_SIZE", 32768.0)])
    _csv(str(d / "cfetch" / "c_counter_collection.csv"), [("copyBuffer", "FETCH_SIZE", 131072.0)])
    _csv(str(d / "cwrite" / "c_counter_collection.csv"), [("copyBuffer", "WRITE_SIZE", 262144.0)])
    out = tmp_path / "ptraffic.txt"
    path, kernels, sources, cmd, what = bench.TRAFFIC["prefill"]
    monkeypatch.setitem(bench.TRAFFIC, "prefill", (str(out), kernels, sources, cmd, what))
    bench.write_traffic_summary("prefill", str(d))
    assert bench.read_traffic("prefill") == pytest.approx((60000.0 * 2.0 + 32768.0) * 1024, rel=1e-6)


def test_cpu_info_names_the_model_and_threads():
    info = bench.cpu_info()
    assert info["nproc"] == os.cpu_count()
    assert 1 <= info["threads"] <= 16 and info["cpu_model"]


def test_busy_summary_round_trip(tmp_path, monkeypatch):
    d = tmp_path / "busy"
    vals = {"SQ_VALU_MFMA_BUSY_CYCLES": 1024 * 300.0, "SQ_BUSY_CYCLES": 1.0, "SQ_WAVE_CYCLES": 1.0,
            "SQ_INSTS_VALU": 2048 * 500.0, "SQ_INSTS_MFMA": 2048 * 64.0, "SQ_INSTS_LDS": 2048 * 40.0,
            "SQ_WAVES": 2048.0, "GRBM_GUI_ACTIVE": 8 * 1000.0, "TCC_HIT_sum": 900.0, "TCC_MISS_sum": 100.0}
    _csv(str(d / "run_counter_collection.csv"), [("prefill_kernel<128>", k, v) for k, v in vals.items()])
    path, kname, sources, cmd = bench.BUSY_FILES["prefill"]
    out = tmp_path / "prefill_counters.txt"
    monkeypatch.setitem(bench.BUSY_FILES, "prefill", (str(out), kname, sources, cmd))
    bench.write_busy_summary("prefill", str(d))
    got = bench.read_busy("prefill")
    # 300 busy cycles per SIMD over 1000 cycles per XCD
    assert got["mfma_busy_frac"] == pytest.approx(0.3)
    assert got["valu_insts_per_wave"] == pytest.approx(500.0)
    assert got["mfma_insts_per_wave"] == pytest.approx(64.0)
    assert got["tcc_hit_rate"] == pytest.approx(0.9)
    out.write_text(out.read_text().replace(bench.source_hash(sources), "0000000000000000"))
    assert bench.read_busy("prefill") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_committed_counter_summaries_match_the_kernel_sources():
    """Every counter-backed summary under profiles/ was taken on the kernel
    sources as they stand: a kernel change without new counters fails here
    (bench.py would otherwise report traffic and busy fractions as null)."""
    for which in ("decode", "prefill"):
        assert bench.read_traffic(which) is not None, f"profiles traffic summary of {which} is stale or missing"
        assert bench.read_busy(which) is not None, f"profiles counter summary of {which} is stale or missing"
