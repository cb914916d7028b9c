"""Host logic of bench.py's rocprofv3 summaries (no GPU): per-kernel means
and the counter normalisations, the HBM traffic record scaled by the copy
calibration, and the trace table with medians."""
import csv
import json
import os

import pytest

import bench

CC_FIELDS = ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value",
             "Start_Timestamp", "End_Timestamp"]
GEMM = "void tfq::(anonymous namespace)::gemm_pipe_kernel<0, 1, true, false, false, 4>(tfq::(anonymous namespace)::Params)"
COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::bfloat16_copy_kernel_cuda>(int)"


def _counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=CC_FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(CC_FIELDS, r)))
    return str(path)


def test_counter_means_and_normalisation(tmp_path, capsys):
    # one dispatch of 1 ms: 8 XCDs at 1.5 GHz, 32 SEs, 1024 SIMDs 60% MFMA-busy
    dur = 1_000_000  # ns
    cyc = 1.5e9 * 1e-3
    rows = [(1, 4096, GEMM, "GRBM_GUI_ACTIVE", 8 * cyc, 0, dur),
            (1, 4096, GEMM, "SQ_CYCLES", 32 * cyc, 0, dur),
            (1, 4096, GEMM, "SQ_VALU_MFMA_BUSY_CYCLES", 0.6 * 1024 * cyc, 0, dur),
            (1, 4096, GEMM, "SQ_BUSY_CYCLES", 0.9 * 32 * cyc, 0, dur),
            (1, 4096, GEMM, "SQ_WAIT_ANY", 25.0, 0, dur),
            (1, 4096, GEMM, "SQ_WAVE_CYCLES", 100.0, 0, dur),
            (1, 4096, COPY, "SQ_CYCLES", 1.0, 0, dur)]
    p = _counters(tmp_path / "a.csv", rows)
    vals, durs = bench.read_counters([p])
    assert list(vals) == ["gemm_pipe_kernel<0, 1, true, false, false, 4> grid=4096"]  # library only
    bench.summarize_counters([p])
    out = capsys.readouterr().out
    line = [l for l in out.splitlines() if l.startswith("| gemm_pipe_kernel")][0]
    cells = [c.strip() for c in line.split("|")[1:-1]]
    assert cells[1] == "1" and cells[2] == "1000.0"
    assert cells[3] == "1.500"   # clock GHz
    assert cells[4] == "0.600"   # MFMA busy
    assert cells[5] == "0.900"   # SQ busy
    assert cells[6] == "0.250"   # wait per wave


def test_traffic_record_scales_by_the_copy(tmp_path, capsys):
    # the copy of 1 GiB reads FETCH_SIZE 2^19 KiB and WRITE_SIZE 2^20 KiB
    cf = _counters(tmp_path / "cf.csv", [(1, 1, COPY, "FETCH_SIZE", 2 ** 19, 0, 1)])
    cw = _counters(tmp_path / "cw.csv", [(1, 1, COPY, "WRITE_SIZE", 2 ** 20, 0, 1)])
    f = _counters(tmp_path / "f.csv", [(1, 4096, GEMM, "FETCH_SIZE", 100.0, 0, 1),
                                       (2, 4096, GEMM, "FETCH_SIZE", 300.0, 0, 1)])
    w = _counters(tmp_path / "w.csv", [(1, 4096, GEMM, "WRITE_SIZE", 50.0, 0, 1)])
    bench.traffic_record(f, w, cf, cw)
    rec = json.loads(capsys.readouterr().out)
    assert rec["fetch_factor"] == 2.0 and rec["write_factor"] == 1.0
    k = rec["kernels"]["gemm_pipe_kernel<0, 1, true, false, false, 4> grid=4096"]
    assert k["read_bytes"] == int(200.0 * 1024 * 2.0) and k["write_bytes"] == 50 * 1024
    for src in ("gemm_source_sha256", "quantize_source_sha256"):
        assert len(rec[src]) == 64


def test_trace_table_has_medians(tmp_path, capsys):
    stats = tmp_path / "x_kernel_stats.csv"
    with open(stats, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs",
                    "MaxNs", "StdDev"])
        w.writerow([GEMM, 3, 9000, 3000, 90.0, 1000, 6000, 0])
        w.writerow([COPY, 1, 1000, 1000, 10.0, 1000, 1000, 0])
    with open(tmp_path / "x_kernel_trace.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for d in (1000, 2000, 6000):
            w.writerow([GEMM, 0, d])
    bench.summarize_trace(str(stats))
    out = capsys.readouterr().out
    line = [l for l in out.splitlines() if "gemm_pipe_kernel" in l][0]
    cells = [c.strip() for c in line.split("|")[1:-1]]
    assert cells[:4] == ["gemm_pipe_kernel<0, 1, true, false, false, 4>", "3", "3.0", "2.0"]
    assert "(other kernels) | 1" in out


def test_measured_traffic_needs_the_same_source(tmp_path, monkeypatch):
    # a record whose hash does not match the kernel source reads as unmeasured
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic_kernel_pass.json").write_text(json.dumps({
        "gemm_source_sha256": "0" * 64, "quantize_source_sha256": "0" * 64,
        "kernels": {"gemm_pipe_kernel<0, 1, true, false, false, 4> grid=4096":
                    {"read_bytes": 1, "write_bytes": 2}}}))
    csrc = tmp_path / "int8_w8a8_quantized_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "gemm.hip").write_text("x")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("gemm_pipe_kernel<0, 1", 4096) is None
    import hashlib
    rec = json.loads((prof / "traffic_kernel_pass.json").read_text())
    rec["gemm_source_sha256"] = hashlib.sha256(b"x").hexdigest()
    (prof / "traffic_kernel_pass.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("gemm_pipe_kernel<0, 1", 4096) == 3
    assert bench.measured_traffic("gemm_pipe_kernel<0, 1", 8192) is None
