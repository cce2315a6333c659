"""The CPU oracle and the C ABI's host code under AddressSanitizer and
UndefinedBehaviorSanitizer.

Two small C drivers (tests/sanitize/) are built with the sanitizers and run:
oracle_check calls every oracle function on small and empty shapes with
exactly sized buffers; abi_check drives the library's argument validation and
plan building (host code only: no call reaches a kernel launch).  The library
is rebuilt for this with the sanitizers on its host code only (device code is
not instrumented), in a temporary directory, at -O1.
"""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from ternary_weight_token_amd import build as libbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CLANG = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang")
SAN = "address,undefined"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_check")
    _run(["gcc", "-O1", "-g", "-std=c11", "-Wall", "-fopenmp", "-ffp-contract=off", f"-fsanitize={SAN}",
          "-fno-sanitize-recover=all", os.path.join(HERE, "oracle_check.c"),
          os.path.join(ROOT, "oracle", "bitnet_oracle.c"), "-o", exe, "-lm"])
    r = _run([exe], env=dict(ENV, OMP_NUM_THREADS="2"), timeout=300)
    assert "checks passed" in r.stdout, r.stdout


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang not available")
def test_abi_host_code_under_sanitizers(tmp_path):
    flags = [f for f in libbuild.FLAGS if f not in ("-O3", "-shared")]
    flags += ["-O1", "-g"] + ["-Xarch_host", f"-fsanitize={SAN}", "-Xarch_host", "-fno-sanitize-recover=all"]
    inc = ["-I", os.path.join(ROOT, "include")]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([libbuild.hipcc(), "-c"] + flags + inc + [os.path.join(libbuild.CSRC, src), "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, libbuild.SOURCES))
    lib = str(tmp_path / "libbitnet_san.so")
    _run([libbuild.hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", f"-fsanitize={SAN}"]
         + objs + ["-o", lib])
    exe = str(tmp_path / "abi_check")
    _run([CLANG, "-O1", "-g", "-std=c11", "-Wall", f"-fsanitize={SAN}", "-fno-sanitize-recover=all"] + inc
         + [os.path.join(HERE, "abi_check.c"), lib, f"-Wl,-rpath,{tmp_path}", "-o", exe])
    r = _run([exe], env=ENV, timeout=300)
    assert "checks passed" in r.stdout, r.stdout
