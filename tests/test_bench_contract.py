"""bench.py's reporting arithmetic and contract, on the CPU (no GPU call).

The figures are checked against values written out by hand from the
workload shapes, not against bench.py's own formulas retyped."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth import WORKLOADS, sweep_points  # noqa: E402


def test_flops_and_bytes_of_the_64k_workload():
    c = WORKLOADS["long_64k"]
    # 4 d B Hq (T(T+1)/2 + T L) = 4*128*16*(65536*65537/2 + 65536*32)
    assert bench.flops(c) == 4 * 128 * 16 * (65536 * 65537 // 2 + 65536 * 32)
    assert abs(bench.flops(c) - 1.761e13) / 1.761e13 < 1e-3
    # bf16: Q and O (2*16*65536*128), K and V (2*4*65536*128), depth (2*4*65536*32*128)
    want = 2 * (2 * 16 * 65536 * 128 + 2 * 4 * 65536 * 128 + 2 * 4 * 65536 * 32 * 128)
    assert bench.fused_bytes(c) == want
    assert abs(want - 4.970e9) / 4.970e9 < 1e-3


def test_roofline_bound_and_fraction():
    c = WORKLOADS["long_64k"]
    r = bench.roofline(c, 14.0, None)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2516.6
    assert r["achieved"] == pytest.approx(bench.flops(c) / 14.0e-3 / 1e12)
    assert r["frac"] == pytest.approx(r["achieved"] / 2516.6)
    # the depth-heavy workload sits below the ridge point (about 315 flop/B): HBM-bound
    d = WORKLOADS["depth_heavy"]
    assert bench.flops(d) / bench.fused_bytes(d) < 2516.6e12 / 8000e9
    r = bench.roofline(d, 4.0, None)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["achieved"] == pytest.approx(bench.fused_bytes(d) / 4.0e-3 / 1e9)


def test_traffic_reported_only_for_the_current_sources(tmp_path, monkeypatch):
    """HBM-traffic figures are reported only while their record names the
    kernel sources as they stand; after a change to those sources, null."""
    (tmp_path / "profiles").mkdir()
    for name, sha in (("fwd_now", bench.kernel_src_hash()), ("fwd_old", "0" * 16)):
        with open(tmp_path / "profiles" / f"{name}_traffic.json", "w") as f:
            json.dump({"kernel_src_sha": sha, "hbm_bytes_per_launch": 123.0}, f)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.load_traffic("fwd_now") == 123.0
    assert bench.load_traffic("fwd_old") is None
    assert bench.load_traffic("fwd_missing") is None


def test_committed_traffic_records_are_plausible():
    """Each committed record reads at least about the workload's algorithmic
    input bytes and writes about O once (bf16)."""
    for w in ("long_64k", "depth_heavy"):
        with open(os.path.join(ROOT, "profiles", f"fwd_{w}_traffic.json")) as f:
            rec = json.load(f)
        c = WORKLOADS[w]
        o_bytes = 2 * c["B"] * c["Hq"] * c["T"] * c["d"]
        assert rec["fetch_bytes"] >= 0.95 * (bench.fused_bytes(c) - o_bytes), w
        assert rec["write_bytes"] == pytest.approx(o_bytes, rel=0.05), w
        assert rec["hbm_bytes_per_launch"] == pytest.approx(rec["fetch_bytes"] + rec["write_bytes"])


def test_cold_timing_selection():
    # cold only where the last-level cache could hold a noticeable share of one call's bytes
    assert bench.cold_cache(WORKLOADS["layer_1p5b"])
    assert not bench.cold_cache(WORKLOADS["long_64k"])
    assert not bench.cold_cache(WORKLOADS["depth_heavy"])
    assert not bench.cold_cache(WORKLOADS["tiny"])
    assert len(sweep_points()) == 36


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode != 0
    assert "one GPU" in p.stderr
    assert p.stdout.strip() == ""
