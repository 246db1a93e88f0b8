"""Host-side logic of bench.py (CPU only): the HBM counter summary, the
algorithmic byte accounting of the launches and the one-GPU refusal."""

import argparse
import csv
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _csv(path, counter, rows):
    """rows: (kernel name, value) in dispatch order."""
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                           "Counter_Value"])
        w.writeheader()
        for i, (k, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": k, "Counter_Name": counter,
                        "Counter_Value": v})


def test_pmc_summary_scales_by_the_copy_calibration(tmp_path):
    # the run ends with three 1 GiB copies (1 GiB read and written each);
    # here the fetch counter shows half of it (factor 2), the write counter
    # all of it (factor 1).  A larger set-up copy earlier in the run is not
    # the calibration.
    kib = (1 << 30) / 1024
    kern, copy = "moe::int8_row_dequant_kernel(...)", "__amd_rocclr_copyBuffer"
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    _csv(f, "FETCH_SIZE", [(copy, 20 * kib), (kern, 1000.0), (kern, 1200.0),
                           (copy, kib / 2), (copy, kib / 2), (copy, kib / 2 + 8)])
    _csv(w, "WRITE_SIZE", [(copy, 40 * kib), (kern, 4000.0), (kern, 4000.0),
                           (copy, kib), (copy, kib), (copy, kib)])
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


def test_one_token_launch_bytes_are_the_layer_s_bytes():
    """The one-token launch runs the whole layer: its algorithmic bytes are
    the three-launch structure's sum less one read of the token (the router
    and the routed gate/up read x in one launch, counted once), and the
    weights in it are exactly the router, 2 shared experts and 16 routed
    experts of the K3 shape."""
    import bench
    one = bench.kernel_bytes("decode_front", 1, 16, 16, 2)
    three = (bench.kernel_bytes("router_shared_gateup_topk", 1, 16, 16, 2)
             + bench.kernel_bytes("shared_down_routed_gateup", 1, 16, 16, 2)
             + bench.kernel_bytes("routed_down_combine", 1, 16, 16, 2))
    assert one == three - 7168 * 2 == 426_093_824
    weights = 896 * 7168 * 2 + 2 * 3 * 7168 * 1536 * 2 + 16 * 17_547_264
    assert weights == 425_721_856
    # activations and intermediates: x twice, logits written and read, ids and
    # weights written and read, h (routed and shared, hi + lo) written and
    # read, the shared outputs written and read, y
    assert one - weights == 371_968


def test_kernel_lists_follow_the_launch_structure():
    """One token: one launch; 2 to 8 tokens: three; more: four; MFMA: five."""
    import bench
    assert bench.config_kernels("b1") == ["decode_front"]
    assert bench.config_kernels("b2") == bench.KERNELS_GEMV_SMALL
    assert bench.config_kernels("b8") == bench.KERNELS_GEMV_SMALL
    assert bench.config_kernels("b64") == bench.KERNELS_GEMV
    assert bench.config_kernels("prefill") == bench.KERNELS_MFMA
