"""bench.py's command-line contract that needs no GPU: a run on more than one
GPU is refused with a message (the path runs on one GPU; there is no
multi-GPU leg), and the help text lists the paths and workloads."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""


def test_help_lists_paths_and_workloads():
    r = run("--help")
    assert r.returncode == 0
    for word in ("deferred", "tree", "fused", "split_neumann", "split_inverse", "multilayer"):
        assert word in r.stdout, word
