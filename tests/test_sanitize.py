"""AddressSanitizer + UBSan builds of the CPU oracle and of the library's host code (no
GPU needed).  Each build links a driver (tests/sanitize/) that exercises every entry point
on the host paths: the oracle on small ragged inputs of both P (its reconstruct, products,
layers and searches), and the library's argument validation, size functions and expert
cache planner.  A sanitizer report or a failed check fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "pseudo_random_weight_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, timeout, env=None):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout, env=env)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stdout[-4000:] + r.stderr[-4000:]
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is needed")
def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-ffp-contract=off",
          "-fopenmp", os.path.join(HERE, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "seedref.c"), "-o", exe, "-lm"], 300)
    out = _run([exe], 300, SAN_ENV)
    assert "clean" in out


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)),
                    reason="the ROCm compilers are needed")
def test_library_host_code_under_address_and_undefined_sanitizers(tmp_path):
    objs = []
    for src in ("seedmm.hip", "search.hip", "expert_cache.hip"):
        obj = str(tmp_path / (src + ".o"))
        # host code instrumented; device code compiled as usual (never run here)
        _run([HIPCC, "-c", "-O1", "-g", "-std=c++17", "--offload-arch=gfx950",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-mllvm", "-disable-promote-alloca-to-lds",
              "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
              "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all",
              "-I", os.path.join(ROOT, "include"), os.path.join(CSRC, src), "-o", obj], 600)
        objs.append(obj)
    exe = str(tmp_path / "host_driver")
    _run([CLANGXX, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
          "-fno-omit-frame-pointer", "-fno-sanitize-recover=all",
          "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "host_driver.cpp"), *objs,
          "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe], 300)
    out = _run([exe], 300, SAN_ENV)
    assert "clean" in out
