"""CPU builds with AddressSanitizer and UndefinedBehaviorSanitizer: the CPU
reference run on small inputs through every function, and the C ABI's host
side (argument checks, workspace sizes, tuning) called with bad arguments.
Only host code is instrumented (the GPU code is compiled as usual)."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def run(cmd, env=None):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr[-4000:]}"
    return r


@pytest.mark.slow
def test_oracle_under_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_driver")
    run(["gcc", "-O1", "-std=c11", "-ffp-contract=off"] + SAN +
        [os.path.join(ROOT, "oracle", "bastion_oracle.c"),
         os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-o", exe, "-lm"])
    r = run([exe], ENV)
    assert "oracle driver ok" in r.stdout


@pytest.mark.slow
def test_abi_host_checks_under_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "abi_driver")
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not os.path.exists(hipcc):
        pytest.skip("hipcc is not installed")
    csrc = os.path.join(ROOT, "block_diffusion_tree_amd", "csrc")
    srcs = [os.path.join(csrc, f) for f in ("api.hip", "build_trees.hip", "tree_ops.hip",
                                            "noalloc.hip", "verify.hip", "stochastic.hip")]
    host_san = []
    for f in SAN:
        host_san += (["-Xarch_host", f] if f.startswith("-fsanitize") or f.startswith("-fno-sanitize")
                     else [f])
    cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-std=c++17", "-ffp-contract=off",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I" + os.path.join(ROOT, "include")] + host_san + srcs + \
          [os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"), "-o", exe]
    run(cmd)
    r = run([exe], ENV)
    assert "abi driver ok" in r.stdout
