"""Builds libw4a16.so for gfx950 with hipcc, in the package directory.

    python -m mixed_precision_w4a16_repack_amd.build

Each source compiles to an object under ``_build/`` (in parallel), then one
shared library is linked next to this file, where the binding loads it.
The sources with MFMA kernels are also compiled to gfx950 assembly:
``wait_check`` verifies the hand-counted memory waits of the staged kernels
against it, and that no MFMA reads an inline-asm VALU result without the
wait states the hardware needs; either problem fails the build.
"""

from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build", "w4a16")
LIB = os.path.join(PKG, "libw4a16.so")
# A plain streaming-read kernel in a library of its own, loaded by the
# benchmark only (the HBM read ceiling of one launch); not part of the path.
CEILING_SRC = "ceiling.hip"
CEILING_LIB = os.path.join(PKG, "libw4a16_ceiling.so")
SOURCES = ["w4a16_api.cpp", "repack.hip", "skinny.hip", "mfma.hip", "dense.hip", "w4a8.hip", "scratch.hip"]
STAGED = ["mfma.hip", "w4a8.hip"]  # kernels with hand-counted waits (wait_check)
ASSEMBLED = STAGED + ["skinny.hip"]  # every source with MFMA kernels (operand hazard check)

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed-fp32 VALU forms are disabled for all device code.
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, "-x", "hip", *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def _assembly(src: str) -> str:
    out = os.path.join(BUILD, os.path.splitext(src)[0] + ".gfx950.s")
    cmd = [HIPCC, "-x", "hip", *FLAGS, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{res.stdout}{res.stderr}")
    return out


def check_waits(asm_paths) -> None:
    """Fails when a staged kernel's hand-counted wait does not match the
    vector-memory instructions the compiler emitted (see wait_check)."""
    from . import wait_check

    problems, kernels = [], 0
    for p in asm_paths:
        with open(p) as f:
            n, probs = wait_check.check_asm(f.read())
        kernels += n
        problems += probs
    if kernels == 0:
        raise RuntimeError("wait check: no staged kernel found in the assembly")
    if problems:
        raise RuntimeError("wait check failed:\n" + "\n".join(problems))


def check_mfma_operands(asm_paths) -> None:
    """Fails when an MFMA reads an inline-asm VALU result too soon (see
    wait_check.mfma_operand_hazards)."""
    from . import wait_check

    problems = []
    for p in asm_paths:
        with open(p) as f:
            problems += wait_check.mfma_operand_hazards(f.read())
    if problems:
        raise RuntimeError("MFMA operand check failed:\n" + "\n".join(problems[:20]))


def _build_ceiling() -> None:
    tmp = CEILING_LIB + ".tmp"
    cmd = [HIPCC, "-x", "hip", *FLAGS, "-shared", os.path.join(CSRC, CEILING_SRC), "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {CEILING_SRC}:\n{res.stdout}{res.stderr}")
    os.replace(tmp, CEILING_LIB)


def build(verbose: bool = False) -> str:
    """Compile every source, check the staged kernels' waits and link
    libw4a16.so. Returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        asm = {s: ex.submit(_assembly, s) for s in ASSEMBLED}
        objs = list(ex.map(_compile, SOURCES))
        asm_paths = {s: f.result() for s, f in asm.items()}
    check_waits([asm_paths[s] for s in STAGED])
    check_mfma_operands(list(asm_paths.values()))
    _build_ceiling()
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, "-L/opt/rocm/lib", "-lhipblaslt"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
