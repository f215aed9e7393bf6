"""Build libbastion.so (gfx950) in-tree with hipcc.

    python -m block_diffusion_tree_amd.build

Each source compiles in its own hipcc process (in parallel) into _build/,
then one link produces block_diffusion_tree_amd/libbastion.so.  The library
depends only on the HIP runtime; it has no PyTorch dependency.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbastion.so")
# the streaming-read ceiling the benchmark measures beside the kernels
PROBE_LIB = os.path.join(PKG, "libbastion_probe.so")
PROBE_SOURCES = ["stream_probe.hip"]
SOURCES = ["api.hip", "build_trees.hip", "tree_ops.hip", "noalloc.hip", "verify.hip",
           "stochastic.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-mcode-object-version=5",
    # no contraction: rho products and S(N) must round exactly as written
    "-ffp-contract=off",
    # no packed fp32 instructions (v_pk_fma/add/mul_f32) anywhere
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I" + os.path.join(ROOT, "include"),
]


def _compile(src: str, outdir: str = None, extra=()) -> str:
    outdir = outdir or BUILD
    obj = os.path.join(outdir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + list(extra) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(line for line in r.stderr.splitlines()
                     if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{errs}")
    if errs.strip():
        sys.stderr.write(errs + "\n")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    if verbose:
        print("built", LIB, "and", PROBE_LIB)
    return LIB


# The stamped library: the same sources compiled with -DBASTION_STAMPS, which
# adds per-block timestamps and bastion_debug_set_stamps (phase tables of
# `python -m block_diffusion_tree_amd.stamps`).  Not the product library.
STAMPS_LIB = os.path.join(PKG, "libbastion_stamps.so")


def build_stamped(verbose: bool = False) -> str:
    out = os.path.join(BUILD, "stamps")
    os.makedirs(out, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda f: _compile(f, out, ["-DBASTION_STAMPS"]), SOURCES))
    _link(objs, STAMPS_LIB)
    if verbose:
        print("built", STAMPS_LIB)
    return STAMPS_LIB


if __name__ == "__main__":
    import sys as _sys
    if "--stamps" in _sys.argv:
        build_stamped(verbose=True)
    else:
        build(verbose=True)
