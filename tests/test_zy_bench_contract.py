"""bench.py's output line on the GPU: one short run of the headline workload
(batch-1 decode, no secondary workloads), checked for the fields a reader of
the line relies on. Collected after the parity tests, so that under `-x` a
failure here hides none of them."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
def test_bench_line_contract():
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "5", "--warmup", "2",
           "--no-secondary", "--cpu-seconds", "2"]
    print("running", " ".join(cmd), flush=True)
    r = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2
    assert d["unit"] == "GB/s" and d["higher_is_better"] is True and d["data"] == "synthetic"
    assert d["config"]["workload"] and "model" not in d["config"]
    assert d["value"] > 0 and d["ms_per_step"] > 0
    # value is the step's algorithmic bytes over its time
    alg = d["config"]["algorithmic_bytes_per_step"]
    assert abs(d["value"] - alg / (d["ms_per_step"] * 1e-3) / 1e9) <= 0.01 * d["value"]
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000
    assert 0 < rf["achieved"] <= rf["peak"]
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    assert cb["nproc"] >= 1 and cb["cpu_model"] and cb["omp_threads"] == cb["cores"]
    # and the same steps on one thread
    one = cb["single_thread"]
    assert one["threads"] == 1 and one["token_steps"] >= 1 and one["value"] > 0
    # a stage that enqueues nothing in this form is null, not a timed empty graph
    assert d["stage_us"]["bucket"] is None and d["stage_us"]["up"] > 0
