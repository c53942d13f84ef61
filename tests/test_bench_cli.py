"""The benchmark's command line on the CPU: a multi-GPU request is refused with a message and a
non-zero status before anything touches a GPU, and the help text lists every workload."""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          cwd=ROOT, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_help_lists_the_workloads():
    r = _run("--help")
    assert r.returncode == 0
    for w in ("layer_decode", "layer_prefill", "layer_skewed", "layer_ep8", "layer_tp8", "gemm_e8_m32"):
        assert w in r.stdout, w
