"""Host logic of bench.py (no GPU): the algorithmic counts the roofline is priced with, the
scaling of the rocprofv3 byte counters by a plain copy, the per-kernel trace table, the
rule that recorded traffic is reported only for the kernel sources it was measured on, and
the one-GPU contract of the command line."""

import csv
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_counts_retention_workload():
    # B4 H8 T2048 d128, chunk 64, bf16: q, k, v read and o written (4 d bf16 per token-head),
    # the final fp32 memory written (d^2 per head); flops over the causal tiles 2d(C + 1) + 4d^2
    # per token-head (the whole-block count 4Cd + 4d^2 beside it)
    flops, bytes_ = bench.algorithmic_counts("retention", 4, 8, 2048, 128, 64)
    th = 4 * 8 * 2048
    assert bytes_ == th * 4 * 128 * 2 + 32 * 128 * 128 * 4 == 69_206_016
    assert flops == th * (2 * 128 * 65 + 4 * 128 * 128) == 5_385_486_336
    assert bench.full_block_flops("retention", 4, 8, 2048, 128, 64) == th * (4 * 64 * 128 + 4 * 128 * 128)


def test_algorithmic_counts_gates():
    th = 2 * 3 * 100
    base = th * 4 * 64 * 2 + 6 * 64 * 64 * 4
    assert bench.algorithmic_counts("retention", 2, 3, 100, 64, 32)[1] == base
    assert bench.algorithmic_counts("mamba2", 2, 3, 100, 64, 32)[1] == base + th * 4        # one gate per token
    assert bench.algorithmic_counts("gla", 2, 3, 100, 64, 32)[1] == base + th * 4 * 64      # one per key channel
    assert bench.algorithmic_counts("gdelta", 2, 3, 100, 64, 32)[1] == base + th * 8        # gate and beta
    # gated delta rule, causal tiles: K K^T strictly lower (C - 1)d, Q K^T, T_U R and P U over the
    # lower triangle 3(C + 1)d, three d x d products 6d^2, the solve 2C^2/3
    flops = bench.algorithmic_counts("gdelta", 2, 3, 100, 64, 32)[0]
    assert flops == pytest.approx(th * (31 * 64 + 3 * 33 * 64 + 6 * 64 * 64 + 2 * 32 * 32 / 3))
    assert bench.full_block_flops("gdelta", 2, 3, 100, 64, 32) == pytest.approx(
        th * (8 * 32 * 64 + 6 * 64 * 64 + 2 * 32 * 32 / 3))


def _counter_csv(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for i, (name, counter, value) in enumerate(rows):
            wr.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_summary_scales_by_the_copy(tmp_path, monkeypatch, capsys):
    """FETCH_SIZE and WRITE_SIZE per dispatch (KiB), averaged over dispatches, scaled by what
    the same counter reads for the 512 MB copy (FETCH_SIZE counts half of the copy's bytes),
    summed over a workload's kernels."""
    k1, k2 = bench.WORKLOAD_KERNELS[bench.MAIN]
    copy_kib = bench.COPY_CAL_MB * 1e6 / 1024
    _counter_csv(tmp_path / "f", [("void " + k1 + "(glr::ck::DspParams)", "FETCH_SIZE", 1000.0),
                                  ("void " + k1 + "(glr::ck::DspParams)", "FETCH_SIZE", 3000.0),
                                  ("void " + k2 + "(glr::ck::DspParams)", "FETCH_SIZE", 100.0)])
    _counter_csv(tmp_path / "w", [("void " + k1 + "(glr::ck::DspParams)", "WRITE_SIZE", 500.0),
                                  ("void " + k2 + "(glr::ck::DspParams)", "WRITE_SIZE", 50.0)])
    _counter_csv(tmp_path / "cf", [("copy_kernel", "FETCH_SIZE", copy_kib / 2), ("copy_kernel", "FETCH_SIZE", 1.0)])
    _counter_csv(tmp_path / "cw", [("copy_kernel", "WRITE_SIZE", copy_kib)])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    bench.summarize_traffic(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"), str(tmp_path / "cw"))
    rec = json.loads(out.read_text())
    assert rec["fetch_scale"] == pytest.approx(2.0)
    assert rec["write_scale"] == pytest.approx(1.0)
    w = rec["workloads"][bench.MAIN]
    assert w["fetch_bytes_per_call"] == pytest.approx((2000.0 + 100.0) * 1024 * 2.0)
    assert w["write_bytes_per_call"] == pytest.approx(550.0 * 1024)
    assert w["hbm_bytes_per_call"] == pytest.approx(2100.0 * 2048 + 550.0 * 1024)
    assert "retention_b4h8_t2048_d128" not in rec["workloads"]   # its kernels did not run
    assert rec["source_sha256"] == bench.kernel_source_hash()
    assert "total per call" in capsys.readouterr().out


def test_mfma_summary(tmp_path, monkeypatch, capsys):
    """MFMA counters per call: MOPS in units of 512 flops, the busy fraction over the chip's
    256 x 4 SIMDs (GPU busy cycles as rocprofv3 reports them, summed over 8 XCDs), summed over
    a workload's kernels."""
    k1, k2 = bench.WORKLOAD_KERNELS[bench.MAIN]
    rows = []
    for k, mops, busy, gui in ((k1, 10.0, 2048.0, 80.0), (k2, 30.0, 6144.0, 80.0)):   # gui summed over 8 XCDs
        rows += [(k, "SQ_INSTS_VALU_MFMA_MOPS_BF16", mops), (k, "SQ_VALU_MFMA_BUSY_CYCLES", busy),
                 (k, "GRBM_GUI_ACTIVE", gui)]
    path = tmp_path / "m"
    os.makedirs(path)
    with open(path / "run_counter_collection.csv", "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for i, (name, counter, value) in enumerate(rows):
            wr.writerow({"Dispatch_Id": i // 3, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})
    out = tmp_path / "mfma.json"
    monkeypatch.setattr(bench, "MFMA_FILE", str(out))
    bench.summarize_mfma(str(path))
    w = json.loads(out.read_text())["workloads"][bench.MAIN]
    assert w["mfma_flop_per_call"] == pytest.approx(40.0 * 512)
    assert w["mfma_busy_frac"] == pytest.approx(8192.0 / (20.0 * 1024))
    assert bench.measured_mfma("no_such_workload") is None


def test_recorded_counters_only_for_the_sources_they_were_measured_on(tmp_path, monkeypatch):
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    assert bench.measured_traffic() is None   # nothing recorded
    rec = {"source_sha256": bench.kernel_source_hash(), "workloads": {bench.MAIN: {"hbm_bytes_per_call": 123.0}}}
    out.write_text(json.dumps(rec))
    assert bench.measured_traffic() == 123.0
    assert bench.measured_traffic("gla_b8h16_t4096_d128") is None
    rec["source_sha256"] = "0" * 64   # the kernel sources changed since
    out.write_text(json.dumps(rec))
    assert bench.measured_traffic() is None


def test_trace_table_groups_by_kernel_and_grid(tmp_path, capsys):
    d = tmp_path / "kt"
    d.mkdir()
    rows = [
        ("void glr::ck::fused_kernel<64, 128, 128, 1, 0>(glr::ck::FusedParams)", 65536, 0, 48000),
        ("void glr::ck::fused_kernel<64, 128, 128, 1, 0>(glr::ck::FusedParams)", 65536, 100000, 150000),
        ("void glr::(anonymous namespace)::vla_kernel<unsigned short, 128, 128, 2>(float)", 131072, 0, 4000000),
        ("void at::native::copy_kernel(int)", 1024, 0, 10),
    ]
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size_X", "Start_Timestamp", "End_Timestamp"])
        wr.writeheader()
        for name, grid, t0, t1 in rows:
            wr.writerow({"Kernel_Name": name, "Grid_Size_X": grid, "Start_Timestamp": t0, "End_Timestamp": t1})
    bench.trace_table(str(d))
    text = capsys.readouterr().out
    assert "| `fused_kernel<64, 128, 128, 1, 0>` | 65536 | 2 | 49.0 | 48.0 | 50.0 |" in text
    assert "| `vla_kernel<unsigned short, 128, 128, 2>` | 131072 | 1 | 4000.0 |" in text
    assert "copy_kernel" not in text   # only library kernels


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, cwd=ROOT, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
