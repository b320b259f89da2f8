"""bench.py's command-line contract that holds without a GPU: it runs on one
GPU only, and says so for any other count."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_exits_with_a_message():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""


def test_help_lists_the_driver_flags():
    r = run_bench("--help")
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--workload", "--prefill", "--new-tokens"):
        assert flag in r.stdout
