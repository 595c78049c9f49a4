"""Build libq4.so for gfx950 (and the host-CPU twin libq4host.so) in-tree.

Usage: ``python -m bit_block_quantized_q4_amd.build`` (or ``build()``).
Every HIP translation unit is compiled with hipcc for ``--offload-arch=gfx950``
in parallel, then linked into ``bit_block_quantized_q4_amd/libq4.so``.  The
build always recompiles; the library is written atomically.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
BUILD_DIR = PKG / "_build"
LIB_PATH = PKG / "libq4.so"
HOST_SRC = PKG / "host" / "q4_host.cpp"
HOST_LIB_PATH = PKG / "libq4host.so"
FLOOR_SRCS = (PKG / "floor" / "q4_read_floor.hip", PKG / "floor" / "q4_mfma_ceiling.hip")
FLOOR_LIB_PATH = PKG / "libq4floor.so"
TRACE_LIB_PATH = PKG / "libq4trace.so"
ARCH = os.environ.get("Q4_OFFLOAD_ARCH", "gfx950")

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-command-line-argument",
    # Disable packed fp32 instructions in device code (v_pk_*_f32).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


# Extra flags per translation unit.  The decode GEMV keeps its small matrix
# products in ordinary VGPRs (no accumulator-register copies); the GEMM keeps
# its large accumulators in AGPRs (the default form).
PER_FILE_FLAGS = {
    "q4_gemv.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "q4_gemv_tile.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _hipcc() -> str:
    cand = os.environ.get("HIPCC")
    if cand:
        return cand
    for p in ("/opt/rocm/bin/hipcc",):
        if os.path.exists(p):
            return p
    return "hipcc"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass warns that it does not know the device-only feature.
    out = "\n".join(
        ln for ln in res.stdout.splitlines()
        if "packed-fp32-ops' is not a recognized feature" not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{out}")
    if out.strip() and verbose:
        print(out, flush=True)


def build_host(verbose: bool = False) -> Path:
    """Compile the host-CPU twin (host/q4_host.cpp, plain C++ with AVX2 code
    behind run-time checks) into libq4host.so; returns its path."""
    cxx = os.environ.get("CXX", "g++")
    tmp = HOST_LIB_PATH.with_suffix(".so.tmp")
    _run([cxx, "-O3", "-std=c++17", "-fPIC", "-shared", "-pthread", "-Wall",
          "-ffp-contract=off", f"-I{INCLUDE}", str(HOST_SRC), "-o", str(tmp)], verbose)
    os.replace(tmp, HOST_LIB_PATH)
    return HOST_LIB_PATH


def build_floor(verbose: bool = False) -> Path:
    """Compile the benchmark's measurement kernels (floor/: the plain read and
    the matrix-core ceiling) into libq4floor.so; returns its path."""
    tmp = FLOOR_LIB_PATH.with_suffix(".so.tmp")
    _run([_hipcc(), *COMMON_FLAGS, "-shared", *map(str, FLOOR_SRCS), "-o", str(tmp)], verbose)
    os.replace(tmp, FLOOR_LIB_PATH)
    return FLOOR_LIB_PATH


def build_trace(verbose: bool = False) -> Path:
    """Link libq4trace.so: libq4's objects with the tile GEMV compiled with
    -DQ4_PHASE_TRACE (its computing waves record per-phase clocks into a
    buffer set by q4_phase_trace_set).  A measurement build for
    `bench.py --phase-trace`; nothing else loads it.  Needs build()'s objects."""
    hipcc = _hipcc()
    src = CSRC / "q4_gemv_tile.hip"
    obj = BUILD_DIR / "q4_gemv_tile_trace.o"
    _run([hipcc, *COMMON_FLAGS, *PER_FILE_FLAGS.get(src.name, []), "-DQ4_PHASE_TRACE",
          "-c", str(src), "-o", str(obj)], verbose)
    objs = [BUILD_DIR / (s.stem + ".o") for s in sorted(CSRC.glob("*.hip")) if s.name != src.name]
    tmp = TRACE_LIB_PATH.with_suffix(".so.tmp")
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp),
          *map(str, objs), str(obj)], verbose)
    os.replace(tmp, TRACE_LIB_PATH)
    return TRACE_LIB_PATH


def build(verbose: bool = False) -> Path:
    """Compile every csrc/*.hip for gfx950 and link libq4.so (and build the
    host-CPU twin libq4host.so and the benchmark's measurement libq4floor.so);
    returns libq4.so's path."""
    build_host(verbose)
    build_floor(verbose)
    hipcc = _hipcc()
    BUILD_DIR.mkdir(exist_ok=True)
    srcs = sorted(CSRC.glob("*.hip"))
    if not srcs:
        raise RuntimeError(f"no HIP sources under {CSRC}")
    objs = [BUILD_DIR / (s.stem + ".o") for s in srcs]
    jobs = min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_run, [hipcc, *COMMON_FLAGS, *PER_FILE_FLAGS.get(s.name, []),
                                 "-c", str(s), "-o", str(o)], verbose)
                for s, o in zip(srcs, objs)]
        for f in futs:
            f.result()
    tmp = LIB_PATH.with_suffix(".so.tmp")
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp),
          *map(str, objs)], verbose)
    os.replace(tmp, LIB_PATH)
    build_trace(verbose)
    return LIB_PATH


if __name__ == "__main__":
    p = build(verbose="-v" in sys.argv)
    print(p)
