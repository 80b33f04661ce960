"""CPU tests of bench.py's argument handling (no GPU: every case here exits
before the benchmark touches a device)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "measures one GPU" in r.stderr and "large_nn_rows" in r.stderr


def test_unknown_workload_is_refused():
    r = run("--workload", "no_such_product")
    assert r.returncode != 0
    assert "unknown workload" in r.stderr and "large_nn_cols8" in r.stderr


def test_bad_sweep_shapes_are_refused():
    for bad in ("4x4", "4x4x0", "axbxc"):
        r = run("--sweep", "--shapes", bad)
        assert r.returncode != 0
        assert "MxNxK" in r.stderr, (bad, r.stderr)


def test_plan_options_need_the_workspace_form():
    r = run("--split-k", "2")
    assert r.returncode != 0
    assert "--workspace" in r.stderr
