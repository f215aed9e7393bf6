"""bench.py's command line and bookkeeping, on the CPU (no GPU call)."""
import os
import subprocess
import sys

import bench
from block_diffusion_tree_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_every_workload_has_a_description():
    for name in list(synth.WORKLOADS) + ["verify"]:
        assert name in bench.WORKLOAD_TEXT, name


def test_defaults_finish_quickly():
    sys_argv = sys.argv
    try:
        sys.argv = ["bench.py"]
        a = bench.parse()
    finally:
        sys.argv = sys_argv
    assert a.gpus == 1 and a.workload == "main"
    assert 1 <= a.steps <= 200 and 0 <= a.warmup <= 20


def test_traffic_is_keyed_by_the_tree_sources():
    csrc = os.path.join(ROOT, "block_diffusion_tree_amd", "csrc")
    for f in bench.TREE_PATH_SOURCES:
        assert os.path.exists(os.path.join(csrc, f)) or os.path.exists(os.path.join(ROOT, "include", f)), f
    h = bench.kernel_source_hash()
    assert h == bench.kernel_source_hash() and len(h) >= 8
