"""bench.py's output contract on a small workload: one JSON line with the
fields the benchmark promises (throughput, roofline entry, configuration)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_json_line_with_the_contract_fields():
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "midvocab_bf16", "--steps", "2",
           "--warmup", "1", "--no-cpu-baseline"]
    print("\n[case] bench.py on the mid-vocab workload", flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [line for line in res.stdout.splitlines() if line.strip()]
    assert len(lines) == 1, res.stdout
    out = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in out, key
    assert out["n_gpus"] == 1 and out["steps"] == 2 and out["warmup"] == 1
    assert out["value"] > 0 and out["ms_per_step"] > 0 and out["unit"] == "TFLOP/s"
    assert out["config"]["workload"].startswith("midvocab_bf16")
    assert "not the headline" in out["metric"]
    roof = out["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert roof["bound"] == "mfma" and 0 < roof["frac"] < 1
    # The library's own memory is the workspace, which never holds an N x V
    # array; everything else the step allocates is an output the caller wanted.
    assert out["workspace_mb"] < out["n_by_v_bytes_mb"]
    assert out["peak_mem_incr_mb"] <= out["workspace_mb"] + out["outputs_mb"] + 1.0


def test_bench_default_warmup_runs_for_a_time():
    """Without --warmup the bench warms for at least 0.5 s and 3 steps and
    reports the count it ran."""
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny_f32", "--steps", "2",
           "--no-cpu-baseline"]
    print("\n[case] bench.py on the tiny workload, default warmup", flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-2000:]
    out = json.loads([line for line in res.stdout.splitlines() if line.strip()][-1])
    # 0.5 s of steps well under 10 ms each
    assert out["warmup"] >= 50 and out["steps"] == 2


def test_bench_one_vocabulary_shard():
    """--vocab-shards: one device's share of a split vocabulary, timed with
    the combine and the shard's backward, reported as its own metric."""
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "midvocab_bf16", "--steps", "2",
           "--warmup", "1", "--no-cpu-baseline", "--vocab-shards", "4", "--shard", "1"]
    print("\n[case] bench.py, shard 1 of 4 of the mid-vocab workload", flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-2000:]
    out = json.loads([line for line in res.stdout.splitlines() if line.strip()][-1])
    assert "one vocabulary shard" in out["metric"] and "not the headline" in out["metric"]
    assert out["config"]["vocab_shard"] == {"offset": 8000, "ids": 8000, "of": 32000, "shards": 4}
    assert out["value"] > 0 and out["roofline"]["traffic"] is None
