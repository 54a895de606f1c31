"""Host sanitizer builds (CPU only): the oracle, and the library's argument
checks, built with AddressSanitizer and UndefinedBehaviorSanitizer and run by
small C drivers (tests/sanitize_oracle.c, tests/sanitize_abi.c). Any
out-of-bounds access, integer overflow or undefined shift aborts a driver.
Only host code is instrumented: the library's device code is compiled
normally, and the ABI driver makes no call that reaches a GPU."""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

from mixed_precision_w4a16_repack_amd import build as lib_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr[-4000:]}"
    return res


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_address_and_undefined_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_driver")
    _run(["gcc", "-std=c99", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fopenmp",
          "-Wall", "-o", exe, os.path.join(ROOT, "oracle", "w4a16_oracle.c"),
          os.path.join(ROOT, "tests", "sanitize_oracle.c"), "-lm"])
    res = _run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=1"))
    assert res.stdout.strip().endswith("ok")


@pytest.mark.skipif(not os.path.exists(lib_build.HIPCC) or shutil.which("gcc") is None, reason="needs hipcc and gcc")
def test_library_argument_checks_under_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    objs = {os.path.splitext(s)[0]: os.path.join(lib_build.BUILD, os.path.splitext(s)[0] + ".o")
            for s in lib_build.SOURCES}
    if not all(os.path.exists(o) for o in objs.values()):
        lib_build.build()
    api = os.path.join(OUT, "w4a16_api_san.o")
    # Host-side instrumentation only: each -fsanitize applies to the host pass.
    _run([lib_build.HIPCC, "-x", "hip", *lib_build.FLAGS, "-O1", "-g", "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all", "-c",
          os.path.join(lib_build.CSRC, "w4a16_api.cpp"), "-o", api])
    drv = os.path.join(OUT, "abi_driver.o")
    _run(["gcc", "-std=c99", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", "-c",
          os.path.join(ROOT, "tests", "sanitize_abi.c"), "-o", drv])
    exe = os.path.join(OUT, "abi_driver")
    others = [o for name, o in objs.items() if name != "w4a16_api"]
    _run([lib_build.HIPCC, f"--offload-arch={lib_build.ARCH}", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
          "-fsanitize=undefined", "-o", exe, drv, api, *others, "-L/opt/rocm/lib", "-lhipblaslt"])
    res = _run([exe], env=ENV)
    assert res.stdout.strip().endswith("ok")
