"""bench.py contract checks that need no GPU."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    """--gpus N with N > 1 exits non-zero with a message saying the run is one-GPU only."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_stored_traffic_matches_the_current_kernel_source():
    """The committed HBM-traffic summary of the prefill GEMM was taken on the
    kernel source as it stands (otherwise bench.py would report traffic null)."""
    with open(os.path.join(ROOT, "profiles", "gemm_w4a4_prefill_traffic.json")) as f:
        d = json.load(f)
    assert d["source_hash"] == bench.kernel_source_hash()
    assert bench.stored_traffic() == d["hbm_bytes_per_launch"]
    M, N, K = d["shape"]
    algorithmic = M * K * 2 + N * K * 0.5625 + 2 * M * N
    assert d["hbm_bytes_per_launch"] >= algorithmic   # the counters cannot see less than the compulsory traffic


def test_stored_mse_lane_ops_match_the_current_kernel_source():
    """The committed VALU counter summary of the MSE search was taken on the
    kernel source as it stands (otherwise bench.py falls back to its op
    model and says so)."""
    with open(os.path.join(ROOT, "profiles", "quantize_mse_valu.json")) as f:
        d = json.load(f)
    assert d["source_hash"] == bench.mse_source_hash()
    assert bench.stored_mse_lane_ops() == d["lane_ops_per_element"] > 16 * 6 / 16
