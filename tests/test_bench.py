"""bench.py's output contract: one JSON line per run with the fields the
benchmark harness reads, in every mode (the product GEMM, sgemm_ws, the
transpose, the ablation ladder).  The GPU runs are short (a few steps) and
run in this process; the argument checks run on the CPU."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KEYS = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
        "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
        "roofline", "cpu_baseline"}
ROOF = {"bound", "achieved", "peak", "unit", "frac", "traffic"}


def run_main(argv, capsys):
    sys.path.insert(0, ROOT)
    import bench
    old = sys.argv
    sys.argv = ["bench.py"] + argv
    try:
        rc = bench.main()
    finally:
        sys.argv = old
    out = capsys.readouterr().out
    lines = [json.loads(l) for l in out.splitlines() if l.startswith("{")]
    return rc, lines


def check_line(d, steps, warmup):
    assert KEYS <= set(d), KEYS - set(d)
    assert ROOF <= set(d["roofline"])
    assert d["n_gpus"] == 1 and d["steps"] == steps and d["warmup"] == warmup
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert 0 < d["roofline"]["frac"] < 1.0
    assert d["roofline"]["achieved"] > 0 and d["data"] == "synthetic"
    assert isinstance(d["config"]["workload"], str)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and not r.stdout.strip()


def test_event_stride_keeps_at_least_ten_samples():
    sys.path.insert(0, ROOT)
    import bench
    for steps in (1, 5, 10, 19, 20, 37, 100, 200, 1000):
        for every in (1, 3, 10, 50):
            k = bench.event_stride(steps, every)
            sampled = [i for i in range(steps) if i % k == k // 2] or [0]
            assert len(sampled) >= min(10, steps), (steps, every)
            assert k <= every


@pytest.mark.gpu
def test_gemm_line(capsys):
    rc, lines = run_main(["--steps", "20", "--warmup", "1", "--workload", "256cube",
                          "--cpu-seconds", "0.05", "--cpu-rows", "256"], capsys)
    assert rc == 0 and len(lines) == 1
    d = lines[0]
    check_line(d, 20, 1)
    assert d["roofline"]["bound"] == "mfma" and d["roofline"]["peak"] == 157.3
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
    assert set(cb["one_core"]) == {"256cube", "ragged"}
    cfg = d["config"]
    assert cfg["event_timed_launches"] >= 10
    assert cfg["clock_ramp_s"] >= 0.3 and cfg["clock_ramp_launches"] >= 20
    # the whole 256^3 product checked against the oracle
    assert cfg["check"]["ok"] and cfg["check"]["elements"] == 256 * 256
    assert 0 <= cfg["max_err_norm"] <= 1e-5
    assert len(cfg["inputs_sha256"]) == 64
    # a matrix-core clock between 1 and 3 GHz, and versions recorded
    assert 1.0 < cfg["clock"]["mfma_clock_ghz"] < 3.0
    assert cfg["versions"]["hip_runtime"] > 0
    # the HBM side of the roofline: compulsory bytes, and the counted bytes
    # when profiles/ holds them for this kernel
    assert 0 < cfg["compulsory_pct_of_hbm_peak"] < 100
    tr = d["roofline"]["traffic"]
    assert (cfg["traffic_hbm_gbs"] is None) == (tr is None)
    if tr is not None:
        assert cfg["traffic_pct_of_hbm_peak"] == pytest.approx(
            100 * cfg["traffic_hbm_gbs"] / 8000, abs=0.02)


@pytest.mark.gpu
def test_split_line(capsys):
    rc, lines = run_main(["--op", "sgemm_ws", "--workload", "256x256x8192",
                          "--steps", "4", "--warmup", "1"], capsys)
    assert rc == 0 and len(lines) == 1
    d = lines[0]
    check_line(d, 4, 1)
    assert d["config"]["splits"] > 1 and d["config"]["workspace_bytes"] > 0


@pytest.mark.gpu
def test_transpose_line(capsys):
    rc, lines = run_main(["--op", "transpose", "--rows", "512", "--cols", "768",
                          "--buffers", "2", "--steps", "3", "--warmup", "1"], capsys)
    assert rc == 0 and len(lines) == 1
    d = lines[0]
    check_line(d, 3, 1)
    assert d["roofline"]["bound"] == "hbm" and d["unit"] == "GB/s"


@pytest.mark.gpu
def test_ladder_lines(capsys):
    rc, lines = run_main(["--ladder", "--workload", "256cube", "--steps", "2",
                          "--warmup", "1"], capsys)
    assert rc == 0 and len(lines) == 14
    for step, d in enumerate(lines):
        check_line(d, 2, 1)
        assert d["config"]["ladder_step"] == step
        assert d["config"]["max_rel_diff_vs_sgemm"] < 1e-5


@pytest.mark.gpu
def test_vendor_lines(capsys):
    rc, lines = run_main(["--op", "vendor", "--shapes", "256x256x256,96x80x4100",
                          "--steps", "3", "--warmup", "1"], capsys)
    assert rc == 0 and len(lines) == 2
    for d, (M, N, K) in zip(lines, [(256, 256, 256), (96, 80, 4100)]):
        assert (d["M"], d["N"], d["K"]) == (M, N, K)
        assert d["sgemm_tflops"] > 0 and d["vendor_tflops"] > 0 and d["sgemm_ws_tflops"] > 0
    assert lines[1]["ws_splits"] > 1
