"""Build libmoe_w8a8.so (gfx950) in-tree with hipcc (one compile per source,
in parallel, then a link).

    python -m moe_expert_ffn_route_amd.build

Flags: -O3; -ffp-contract=off so every fp32 multiply and add of the epilogues
is a separately rounded IEEE operation (no FMA contraction); packed-fp32
instructions disabled on the device side.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe_w8a8.so")
SOURCES = ["abi.hip", "route.hip", "quant.hip", "gemm.hip", "gemm_wide.hip", "gemm_tall.hip", "gemm_mx.hip", "combine.hip",
           "pack.hip", "warm.hip"]
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}", "-ffp-contract=off",
         "-fno-fast-math", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-fvisibility=hidden", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{errs}")
    if errs.strip() and verbose:
        print(errs, file=sys.stderr)


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every HIP source into the shared library (always rebuilds):
    one hipcc per source, in parallel, then one link. Every kernel is launched
    from the source that defines it, so no relocatable device code is needed."""
    import shutil
    import tempfile
    from concurrent.futures import ThreadPoolExecutor

    obj_dir = tempfile.mkdtemp(prefix="moe_w8a8_build_")
    try:
        cflags = [f for f in FLAGS if f != "-shared"]
        objs = [os.path.join(obj_dir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        cmds = [[HIPCC, *cflags, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
        jobs = jobs or max(1, min(len(cmds), os.cpu_count() or 1, 16))
        with ThreadPoolExecutor(jobs) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
        tmp = LIB + f".tmp{os.getpid()}"
        _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp], verbose)
        os.replace(tmp, LIB)
    finally:
        shutil.rmtree(obj_dir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
