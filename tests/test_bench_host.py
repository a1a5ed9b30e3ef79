"""Host logic of bench.py, without a GPU: the one-GPU refusal, kernel-name shortening, the kernel-trace
summary, and the HBM-traffic records (counter bytes scaled by the calibration copy, reported only for
the workload and the kernel sources they were taken on)."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


@pytest.mark.parametrize("name,short", [
    ("_ZN2fg15rowstats_kernelIDF16bLi128EEEvPKT_S3_PfS4_P15HIP_vector_typeIfLj2EEiiiiif", "rowstats_kernel"),
    ("_ZN2fg22decode_partials_kernelIDF16bLi128ELi1EEEvPKT_PfPKiS3_S3_S6_iif", "decode_partials_kernel"),
    ("void fg::gather_kernel<__bf16, 128, 64>(__bf16 const*, __bf16 const*)", "gather_kernel"),
    ("__amd_rocclr_copyBuffer", "__amd_rocclr_copyBuffer"),
])
def test_kernel_names_are_shortened(name, short):
    assert bench._short(name) == short


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_trace_summary_counts_and_averages(tmp_path):
    rows = [["_ZN2fg14colsums_kernelIDF16bLi128ELb0EEEvPKT_", 1000, 1600],
            ["_ZN2fg14colsums_kernelIDF16bLi128ELb0EEEvPKT_", 2000, 3000],
            ["_ZN2fg13select_kernelILi2ELi512EEEvPf", 5000, 5020]]
    _write_csv(str(tmp_path / "run" / "t_kernel_trace.csv"), ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    text = bench.summarize_trace(str(tmp_path), "title", "cmd")
    line = next(x for x in text.splitlines() if x.startswith("colsums_kernel"))
    calls, avg, lo, hi = line.split()[1:5]
    assert int(calls) == 2 and float(avg) == pytest.approx(0.8) and float(lo) == pytest.approx(0.6)
    assert float(hi) == pytest.approx(1.0)
    assert any(x.startswith("select_kernel") for x in text.splitlines())


def test_traffic_records_scale_by_the_calibration_copy(tmp_path, monkeypatch):
    traffic = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(traffic))
    calib_grid = bench.CALIB_BLOCKS * 256
    head = ["Kernel_Name", "Counter_Name", "Counter_Value", "Grid_Size"]
    calib_kib = bench.CALIB_BYTES / 1024
    # the calibration copy reads half of its bytes in FETCH_SIZE and all of them in WRITE_SIZE
    _write_csv(str(tmp_path / "f" / "p_counter_collection.csv"), head,
               [["_ZN2fg16peak_copy_kernelILb0EEEvPK15HIP_vector_type", "FETCH_SIZE", calib_kib / 2, calib_grid],
                ["_ZN2fg22decode_partials_kernelIDF16bLi128ELi1EEEvPKT_", "FETCH_SIZE", 1000.0, 512],
                ["_ZN2fg22decode_partials_kernelIDF16bLi128ELi1EEEvPKT_", "FETCH_SIZE", 3000.0, 512]])
    _write_csv(str(tmp_path / "w" / "p_counter_collection.csv"), head,
               [["_ZN2fg16peak_copy_kernelILb0EEEvPK15HIP_vector_type", "WRITE_SIZE", calib_kib, calib_grid],
                ["_ZN2fg22decode_partials_kernelIDF16bLi128ELi1EEEvPKT_", "WRITE_SIZE", 10.0, 512]])
    text = bench.record_traffic(str(tmp_path / "f"), str(tmp_path / "w"), "wl", "cmd")
    want = 2000.0 * 1024 * 2.0 + 10.0 * 1024 * 1.0            # mean FETCH x 2 + mean WRITE x 1
    assert "decode_partials_kernel" in text
    assert bench.measured_traffic("decode_partials", "wl") == pytest.approx(want)
    assert bench.measured_traffic("decode_partials", "another workload") is None
    assert bench.measured_traffic("profile_rowstats", "wl") is None       # not recorded
    monkeypatch.setattr(bench, "kernel_sources_digest", lambda kernel=None: "other sources")
    assert bench.measured_traffic("decode_partials", "wl") is None        # taken on other sources
