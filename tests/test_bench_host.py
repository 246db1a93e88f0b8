"""Host-side logic of bench.py (CPU only): the HBM counter summary and the
one-GPU refusal."""

import argparse
import csv
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _csv(path, counter, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for k, vals in rows.items():
            for v in vals:
                w.writerow({"Kernel_Name": k, "Counter_Name": counter, "Counter_Value": v})


def test_pmc_summary_scales_by_the_copy_calibration(tmp_path):
    # a 1 GiB copy reads 1 GiB and writes 1 GiB; here the fetch counter shows
    # half of it (factor 2), the write counter all of it (factor 1)
    kib = (1 << 30) / 1024
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    _csv(f, "FETCH_SIZE", {"moe::int8_row_dequant_kernel(...)": [1000.0, 1200.0],
                           "__amd_rocclr_copyBuffer": [kib / 2, 10.0]})
    _csv(w, "WRITE_SIZE", {"moe::int8_row_dequant_kernel(...)": [4000.0, 4000.0],
                           "__amd_rocclr_copyBuffer": [kib]})
    args = argparse.Namespace(config="int8_dequant", pmc_summary=[str(f), str(w)])
    out = bench.pmc_summary(args, out_dir=str(tmp_path))
    assert out["calibration"]["fetch_scale"] == 2.0 and out["calibration"]["write_scale"] == 1.0
    assert out["fetch_bytes_per_launch"] == round(1100.0 * 1024 * 2)
    assert out["write_bytes_per_launch"] == 4000 * 1024
    assert out["bytes_per_launch"] == out["fetch_bytes_per_launch"] + out["write_bytes_per_launch"]
    c = bench.CONFIGS["int8_dequant"]
    assert out["algorithmic_bytes"] == c["rows"] * c["cols"] * 5 + c["rows"] * 4
    assert out["source_hash"] == bench.source_hash()
    assert (tmp_path / "pmc_int8_row_dequant_int8_dequant.json").exists()


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
