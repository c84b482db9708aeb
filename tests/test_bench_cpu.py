"""bench.py's contract, checked without a GPU: it measures one GPU only (any
--gpus above 1 exits with a message saying so), and without a GPU it stops
instead of timing anything else."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    env = dict(os.environ, HIP_VISIBLE_DEVICES="")   # no device, even on a GPU machine
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, env=env)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run_bench("--gpus", "2")
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr


def test_without_a_gpu_nothing_is_timed():
    r = run_bench("--steps", "1", "--warmup", "0", "--cpu-seconds", "0")
    assert r.returncode != 0
    assert "needs a GPU" in r.stdout + r.stderr
    assert '"metric"' not in r.stdout
