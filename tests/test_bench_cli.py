"""bench.py's command line on the host: it measures one GPU and says so when
asked for more (no GPU needed: it exits before importing torch)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                       cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_bench_refuses_a_multi_rank_launch():
    env = dict(os.environ, WORLD_SIZE="2")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_bench_refuses_both_idot_forms():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "prefill_4096_idot",
                        "--idot-int8", "--idot-bf16"], cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "different forms" in r.stderr
    assert r.stdout == ""
