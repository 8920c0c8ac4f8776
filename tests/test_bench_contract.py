"""bench.py's contract, checked without a GPU.

* --gpus N > 1 exits with a message and prints no result line;
* with no GPU visible it fails loudly instead of printing a number;
* the roofline `traffic` figure is read from the committed profile only
  while the GEMM source is the one the counters were taken on;
* the cpu_baseline object carries the keys the report needs.
"""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_exits_with_a_message():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_no_gpu_fails_loudly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    r = run_bench("--steps", "1", "--warmup", "0", "--no-cpu-baseline")
    assert r.returncode != 0
    assert "needs a GPU" in (r.stdout + r.stderr)
    assert not any(line.startswith("{") for line in r.stdout.splitlines())


def test_traffic_only_for_the_profiled_source(tmp_path, monkeypatch):
    v = bench.gemm_traffic_per_launch()
    assert v is not None and v > 0      # the committed profile matches the source
    src = open(bench.GEMM_SRC, "rb").read()
    commented = tmp_path / "commented.hip"
    commented.write_bytes(src + b"\n// a comment\n   \n")
    monkeypatch.setattr(bench, "GEMM_SRC", str(commented))
    assert bench.gemm_traffic_per_launch() == v   # comments do not change the code
    changed = tmp_path / "changed.hip"
    changed.write_bytes(src.replace(b"constexpr int STAGES = 4;", b"constexpr int STAGES = 5;"))
    monkeypatch.setattr(bench, "GEMM_SRC", str(changed))
    assert bench.gemm_traffic_per_launch() is None


def test_cpu_baseline_keys():
    out = bench.cpu_baseline(1, (2,), 1.0)      # the 256 x 1024 workload: a fraction of a second
    for key in ("value", "unit", "cores", "kind", "sample"):
        assert key in out
    assert out["kind"] == "oracle" and out["unit"] == "matrices/s"
    assert out["value"] > 0 and out["cores"] >= 1
    json.dumps(out)


def test_pages_flop_count():
    """The pages' Gram flop count per call (SYRK at s(s+1)l, Q X at 2s^2 l,
    s^3 products at 2s^3; 14 of them for restarts [2], 11 for [1, 3]) on
    three workloads, against the closed form evaluated by hand."""
    def closed(s, l, r, m3):
        return (1 + r) * s * (s + 1) * l + (1 + r) * 2 * s * s * l + m3 * 2 * s ** 3
    assert bench.pages_flops([(256, 1024)], 5, (2,)) == closed(256, 1024, 1, 14)
    assert bench.pages_flops([(8192, 2048)], 5, (1, 3)) == closed(2048, 8192, 2, 11)
    llama = [(4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096),
             (14336, 4096), (14336, 4096), (4096, 14336)] * 4
    want = sum(closed(min(s), max(s), 1, 14) for s in llama)
    assert bench.pages_flops(llama, 5, (2,)) == want
    assert abs(want / 1e12 - 59.547) < 1e-3
    # restart 0 and out-of-range indices are no restarts
    assert bench.pages_flops([(64, 64)], 5, (0,)) == closed(64, 64, 0, 5 + 4 + 8)


def test_oracle_flop_count():
    """fp64 flops of one oracle gram call: full products everywhere, so the
    Gram R = X X^T at 2 s^2 l (once plus once per effective restart), the
    Q X products at 2 s^2 l, and 14 s^3 products for five steps with a
    restart before step 2 (5 Z, 3 Q updates, 3 recurrences of two), 11 for
    restarts [1, 3]."""
    s, l = 256, 1024
    assert bench.oracle_gram_flops(s, l, 5, (2,)) == 2 * (2 * s * s * l) * 2 + 14 * 2 * s ** 3
    assert bench.oracle_gram_flops(s, l, 5, (1, 3)) == 3 * (2 * s * s * l) * 2 + 11 * 2 * s ** 3
    assert bench.oracle_gram_flops(s, l, 5, ()) == 1 * (2 * s * s * l) * 2 + 17 * 2 * s ** 3


def test_target_is_stated_on_work_done():
    import workloads as W
    t = bench.target_status(1086.0, 28, W.WORKLOADS[4], 37.0, 5)
    assert abs(t["pct_fp16_peak_work_done"] - 43.44) < 1e-6
    assert t["met"] is False and t["target_pct_fp16_peak"] == 50.0
    assert "value_over_target" not in json.dumps(t)
