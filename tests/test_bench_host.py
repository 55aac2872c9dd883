"""Host-side parts of bench.py: the HBM-traffic summary built from rocprofv3
counter files, the source-hash gate that keeps a stale summary out of the
JSON line, and the refusal of more than one GPU."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
          "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
          "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
          "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _write_csv(path, counter, rows):
    """rows: (kernel name, [values]) per dispatch; several values become
    several rows of the same dispatch (as for per-dimension counters)."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for d, (name, vals) in enumerate(rows, start=1):
            for v in vals:
                w.writerow({k: 0 for k in FIELDS} | {
                    "Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter,
                    "Counter_Value": f"{v:.6f}"})


def _probe_rows(gemm_vals, copy_val, fill_val):
    rows = [("__amd_rocclr_copyBuffer", [999.0])]          # a set-up copy
    for i in range(6):
        for M in bench.MS:
            rows.append((f"void (anonymous namespace)::k_gemm_km<{M}, 4, 0>(GemmArgs)",
                         gemm_vals[M]))
    rows.append(("void at::native::vectorized_elementwise_kernel<16>", [fill_val]))
    rows.append(("__amd_rocclr_copyBuffer", [copy_val]))
    return rows


@pytest.fixture
def traffic_file(tmp_path, monkeypatch):
    path = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    return path


def test_traffic_summary_scales_by_the_copy(tmp_path, traffic_file):
    copy_kib = bench.COPY_BYTES / 1024
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    # FETCH_SIZE reads the copy at half its size (scale 2); per-dimension rows are summed
    _write_csv(fetch, "FETCH_SIZE", _probe_rows({1: [6000.0, 4000.0], 16: [12000.0]},
                                                copy_kib / 2, 5.0))
    _write_csv(write, "WRITE_SIZE", _probe_rows({1: [28.0], 16: [448.0]}, copy_kib, copy_kib))
    assert bench.traffic_summary(str(fetch), str(write)) == 0
    t = json.loads(traffic_file.read_text())
    assert t["kernel_source_sha256_16"] == bench.kernel_source_hash()
    assert t["fetch_scale"] == pytest.approx(2.0)
    assert t["write_scale"] == pytest.approx(1.0)
    m1, m16 = t["per_m"]["1"], t["per_m"]["16"]
    assert m1["kernel"] == "k_gemm_km<1, 4, 0>" and m1["dispatches"] == 6
    assert m1["hbm_bytes_per_launch"] == round(10000 * 1024 * 2 + 28 * 1024)
    assert m16["hbm_bytes_per_launch"] == round(12000 * 1024 * 2 + 448 * 1024)
    assert m1["algorithmic_bytes"] == bench.algorithmic_bytes(1, bench.N_, bench.K_, bench.G_)
    # the gate: the JSON line carries the bytes only while the source hash matches
    assert bench._traffic(1) == pytest.approx(m1["hbm_bytes_per_launch"])
    t["kernel_source_sha256_16"] = "0" * 16
    traffic_file.write_text(json.dumps(t))
    assert bench._traffic(1) is None


def test_traffic_summary_needs_the_calibration_copy(tmp_path, traffic_file):
    fetch = tmp_path / "fetch.csv"
    rows = _probe_rows({1: [1.0], 16: [1.0]}, 1.0, 1.0)[:-1]   # no closing copy
    _write_csv(fetch, "FETCH_SIZE", rows)
    _write_csv(tmp_path / "write.csv", "WRITE_SIZE", rows)
    with pytest.raises(SystemExit):
        bench.traffic_summary(str(fetch), str(tmp_path / "write.csv"))
    assert not traffic_file.exists()


def test_more_than_one_gpu_is_refused():
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
