"""Address and undefined-behaviour sanitizer builds (host code only, on the CPU).

1. The oracle, built with gcc -fsanitize=address,undefined, driven by
   tests/sanitize/oracle_driver.c over every oracle function on ragged inputs.
2. The library's host code (argument validation of every entry point), built
   with the same sanitizers on the host side only (device code is compiled
   normally and never launched), driven by tests/sanitize/abi_driver.cpp with
   invalid and extreme arguments -- every call is rejected before any launch.

Any out-of-bounds access, leak or signed overflow aborts the driver.
"""
import concurrent.futures
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "video_diffusion_transformer_h3f_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SOURCES = ["api", "k_elementwise", "k_adaln", "k_qk_rope", "k_reduce", "k_router"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "oracle"),
          os.path.join(ROOT, "oracle", "h3oracle.c"), os.path.join(SAN, "oracle_driver.c"),
          "-o", exe, "-lm"])
    r = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1", OMP_NUM_THREADS="2"))
    assert "oracle sanitizer run: ok" in r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)),
                    reason="ROCm compilers not available")
def test_validation_under_asan_ubsan(tmp_path):
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all"]

    def compile_one(name):
        obj = str(tmp_path / f"{name}.o")
        _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san,
              "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, f"{name}.hip"),
              "-o", obj])
        return obj

    with concurrent.futures.ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    drv = str(tmp_path / "driver.o")
    _run([CLANGXX, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-c",
          os.path.join(SAN, "abi_driver.cpp"), "-o", drv])
    exe = str(tmp_path / "abi_driver")
    # link line: no -Xarch_ option, so device sanitizing is switched off explicitly
    _run([HIPCC, "--offload-arch=gfx950", "-fsanitize=address", "-fno-gpu-sanitize",
          "-fsanitize=undefined", drv, *objs, "-o", exe])
    r = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"))
    assert "abi sanitizer run: ok" in r.stdout
