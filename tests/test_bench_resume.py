"""Resumable sweep results (bench.py --sweep --results FILE), on the CPU."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_results_file_round_trip(tmp_path, capsys):
    path = str(tmp_path / "sweep.jsonl")
    assert bench.finished_points(path) == set()
    assert bench.finished_points(None) == set()
    bench.emit_point(path, {"config": "sweep_T4096_L0_G1", "fwd_ms": 0.08})
    bench.emit_point(path, {"config": "sweep_T4096_L8_G1", "fwd_ms": 0.15})
    out = capsys.readouterr().out.splitlines()
    assert [json.loads(l)["config"] for l in out] == ["sweep_T4096_L0_G1", "sweep_T4096_L8_G1"]
    assert bench.finished_points(path) == {"sweep_T4096_L0_G1", "sweep_T4096_L8_G1"}
    # a run killed mid-write leaves a truncated last line: that point counts as unfinished
    with open(path, "a") as f:
        f.write('{"config": "sweep_T4096_L32_G1", "fwd')
    assert bench.finished_points(path) == {"sweep_T4096_L0_G1", "sweep_T4096_L8_G1"}
    # the next point's line starts on a line of its own
    bench.emit_point(path, {"config": "sweep_T4096_L96_G1", "fwd_ms": 0.4})
    assert bench.finished_points(path) == {"sweep_T4096_L0_G1", "sweep_T4096_L8_G1",
                                           "sweep_T4096_L96_G1"}
    # every name the sweep can skip is a sweep point's name
    names = {c["name"] for c in __import__("synth").sweep_points()}
    assert bench.finished_points(path) <= names
