"""Host-side AddressSanitizer / UndefinedBehaviorSanitizer builds (CPU only).

* The CPU oracle (plain C) is built with gcc -fsanitize=address,undefined and
  every function is driven on small and edge-case shapes
  (tests/sanitize/oracle_driver.c).
* The library's sources are built with the sanitizers on their host code
  (each -fsanitize= after -Xarch_host: the device code is compiled as usual and
  never run) and every entry point's argument validation plus every
  compute-free helper is driven without a GPU (tests/sanitize/abi_driver.cpp).

Any sanitizer report aborts the driver (-fno-sanitize-recover=all), so the
tests pass only if every access and integer operation on those paths is clean.
"""
import concurrent.futures as cf
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "bitlinear_matmul_02_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-4000:], r.stderr[-4000:])
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          "-Wall", "-Wextra", "-o", exe, os.path.join(SAN, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "bitlinear_oracle.c"), "-lm"])
    r = _run([exe], env=ENV, timeout=300)
    assert "all checks passed" in r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_abi_validation_under_asan_ubsan(tmp_path):
    flags = ["-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-ffp-contract=off",
             "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    srcs = [os.path.join(CSRC, f) for f in
            ("abi.cpp", "gemv.hip", "gemm.hip", "quant_act.hip", "pack.hip", "glue.hip", "train.hip",
             "noalloc.hip")]
    srcs.append(os.path.join(SAN, "abi_driver.cpp"))

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC, *flags, "-c", src, "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(min(len(srcs), max(1, os.cpu_count() or 1))) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "abi_driver")
    _run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
          "-fsanitize=undefined", "-o", exe, *objs])
    r = _run([exe], env=ENV, timeout=300)
    assert "all checks passed" in r.stdout
