"""bench.py's command line on a machine without a GPU: more than one GPU is
refused with a message, and the workload names it accepts are the
synthetic workloads."""
import os
import subprocess
import sys

from token_activation_perturbation_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    res = run("--gpus", "2")
    assert res.returncode != 0
    assert "one GPU" in (res.stdout + res.stderr)


def test_unknown_workload_is_refused():
    res = run("--workload", "no_such_workload", "--cpu-budget", "0")
    assert res.returncode != 0
    assert "unknown workload" in res.stderr and "bf16_layer" in res.stderr


def test_default_workload_is_the_benchmarked_layer():
    assert "bf16_layer" in synth.WORKLOADS
    src = open(os.path.join(ROOT, "bench.py")).read()
    assert 'default="bf16_layer"' in src or "default='bf16_layer'" in src
