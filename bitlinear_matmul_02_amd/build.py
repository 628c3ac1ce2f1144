"""Build libbitlinear.so (HIP, gfx950 only) in-tree.

    python -m bitlinear_matmul_02_amd.build

Every source is compiled by hipcc for gfx950 with no fast-math, no floating
point contraction, correctly rounded fp32 division, and packed-fp32 ALU ops
disabled; the objects are linked into bitlinear_matmul_02_amd/lib/.

A second library, libbitlinear_lds_poison.so, is the same sources built with
-DBL_LDS_POISON: its kernels poison their LDS before first use (and the
prefill GEMM each consumed staging buffer), a self-test of the barriers and
offsets that the GPU tests run against the oracle.  Nothing else loads it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB_DIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIB_DIR, "libbitlinear.so")
POISON_LIB = os.path.join(LIB_DIR, "libbitlinear_lds_poison.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-x", "hip", "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC,
]
SOURCES = ["abi.cpp", "quant_act.hip", "pack.hip", "gemv.hip", "gemm.hip", "glue.hip", "train.hip", "noalloc.hip"]


def _compile(src: str, build_dir: str = BUILD, extra: tuple = ()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def _link(objs: list, lib: str) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False, poison: bool = True) -> str:
    """Build libbitlinear.so and (poison=True) the LDS self-test library."""
    variants = [(BUILD, (), LIB)]
    if poison:
        variants.append((BUILD + "_lds_poison", ("-DBL_LDS_POISON",), POISON_LIB))
    for d, _, _ in variants:
        os.makedirs(d, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    jobs = max(1, min(8, os.cpu_count() or 1))
    work = [(src, d, extra) for d, extra, _ in variants for src in SOURCES]
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda w: _compile(*w), work))
    for i, (_, _, lib) in enumerate(variants):
        _link(objs[i * len(SOURCES):(i + 1) * len(SOURCES)], lib)
        if verbose:
            print("built", lib)
    return LIB


if __name__ == "__main__":
    build(verbose=True, poison="--no-poison" not in sys.argv)
    sys.exit(0)
