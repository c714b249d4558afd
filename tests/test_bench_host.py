"""Host-side checks of bench.py (no GPU): it refuses more than one GPU, and
the committed HBM counter summary of the headline kernel belongs to the
prefill sources as they stand (bench.py reports its traffic as null
otherwise), with algorithmic bytes equal to the headline workload's tensors
(1 x 16384 tokens, 16 heads, d 128, bf16 Q/K/V/O, fp32 LSE)."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _traffic_values():
    vals = {}
    with open(bench.TRAFFIC_FILE) as f:
        for ln in f:
            if "=" in ln and not ln.startswith("#"):
                k, v = ln.split("=", 1)
                vals[k.strip()] = v.strip()
    return vals


def test_traffic_summary_matches_kernel_sources():
    vals = _traffic_values()
    assert vals["kernel_hash"] == bench.kernel_hash()
    assert bench.read_traffic() == float(vals["hbm_bytes_per_launch"])


def test_traffic_summary_arithmetic():
    vals = _traffic_values()
    tokens, heads, d = 16384, 16, 128
    assert int(vals["algorithmic_read_bytes"]) == 3 * tokens * heads * d * 2
    assert int(vals["algorithmic_write_bytes"]) == tokens * heads * d * 2 + tokens * heads * 4
    fetch = float(vals["fetch_kib_per_dispatch_raw"]) * 1024 * float(vals["fetch_scale"])
    write = float(vals["write_kib_per_dispatch_raw"]) * 1024 * float(vals["write_scale"])
    assert abs(fetch - int(vals["fetch_bytes_per_launch"])) <= 1e-3 * fetch
    assert abs(write - int(vals["write_bytes_per_launch"])) <= 1e-3 * write
    assert int(vals["hbm_bytes_per_launch"]) == int(vals["fetch_bytes_per_launch"]) + int(vals["write_bytes_per_launch"])
