"""Host-side checks of bench.py (no GPU): it refuses more than one GPU, its
closed-form visible-pair counts agree with the oracle's dense masks, and each
committed counter summary belongs to the kernel sources as they stand
(bench.py reports its traffic as null otherwise), with algorithmic bytes
equal to its workload's tensors."""

import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402
from oracle import masks as OM  # noqa: E402


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_visible_pair_counts_match_dense_masks():
    # block mask with triangles, at a reduced shape and at the full one
    for q, k, dk, nb, blk in ((900, 700, 512, 5, 30), (32768, 29576, 24576, 50, 100)):
        n = bench.block_triangle_unmasked(q, dk, nb, blk)
        if q < 1000:
            m = OM.ranges(q, k, W.gen.block_triangle_ranges(q, k, dk, nb, blk))
            assert n == int(m.sum())
        else:
            assert n == 805558868
    assert bench.causal_unmasked(32768, 29576) == 29576 * 29577 // 2
    assert bench.causal_unmasked(300, 700) == int(OM.causal(300, 700).sum())
    assert bench.chunk_unmasked(600, 64, 2) == int(OM.ranges(600, 600, W.gen.chunk_ranges(600, 64, 2)).sum())


def _summary(path):
    vals = {}
    with open(path) as f:
        for ln in f:
            if "=" in ln and not ln.startswith("#"):
                k, v = ln.split("=", 1)
                vals[k.strip()] = v.strip()
    return vals


TRAFFIC = [
    # (file, tokens q, kv, hq, hkv, d)
    (bench.TRAFFIC_FILE, 32768, 29576, 32, 8, 128),
    (bench.TRAFFIC_FILE_CFG4, 16384, 16384, 16, 16, 128),
]


@pytest.mark.parametrize("path,q,kv,hq,hkv,d", TRAFFIC)
def test_traffic_summary_arithmetic(path, q, kv, hq, hkv, d):
    if not os.path.exists(path):
        pytest.skip("no committed summary")
    vals = _summary(path)
    assert int(vals["algorithmic_read_bytes"]) == (q * hq + 2 * kv * hkv) * d * 2
    assert int(vals["algorithmic_write_bytes"]) == q * hq * d * 2 + q * hq * 4
    fetch = float(vals["fetch_kib_per_dispatch_raw"]) * 1024 * float(vals["fetch_scale"])
    write = float(vals["write_kib_per_dispatch_raw"]) * 1024 * float(vals["write_scale"])
    assert abs(fetch - int(vals["fetch_bytes_per_launch"])) <= 1e-3 * fetch
    assert abs(write - int(vals["write_bytes_per_launch"])) <= 1e-3 * write
    assert int(vals["hbm_bytes_per_launch"]) == int(vals["fetch_bytes_per_launch"]) + int(vals["write_bytes_per_launch"])
    if vals["kernel_hash"] == bench.kernel_hash():
        assert bench.read_traffic(path) == float(vals["hbm_bytes_per_launch"])
    else:
        assert bench.read_traffic(path) is None


def test_counters_summary_arithmetic():
    for path in (bench.COUNTERS_FILE, bench.COUNTERS_FILE_CFG4):
        if not os.path.exists(path):
            continue
        v = _summary(path)
        busy = float(v["sq_valu_mfma_busy_cycles"])
        gui = float(v["grbm_gui_active"])
        assert abs(float(v["mfma_busy_pct"]) - 100 * busy / (gui / 8 * 1024)) < 0.05
        flops = 512 * float(v["sq_insts_valu_mfma_mops_bf16"])
        assert abs(float(v["mfma_flops_executed"]) - flops) <= 1e-5 * flops
