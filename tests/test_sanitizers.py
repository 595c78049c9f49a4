"""Host-side code under sanitizers (no GPU): the host-CPU twin (libq4host)
under AddressSanitizer + UndefinedBehaviorSanitizer and under
ThreadSanitizer (its std::thread pool), and libq4's host code (argument
checks, size helpers, the GEMM launch planner) under AddressSanitizer +
UndefinedBehaviorSanitizer.  Each builds a sanitized driver from the
library's own sources (tests/sanitize/*.cpp) in a temporary directory and runs
it; any sanitizer report, or a wrong result, fails the test."""

import os
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
PKG = ROOT / "bit_block_quantized_q4_amd"
HOST_SRC = PKG / "host" / "q4_host.cpp"
DRIVERS = Path(__file__).resolve().parent / "sanitize"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
GXX = shutil.which("g++")

ENV = dict(os.environ,
           ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1:exitcode=71",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=72",
           TSAN_OPTIONS="halt_on_error=1:exitcode=73")


def run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    return r.returncode, r.stdout


def build_and_run(cmd, exe):
    rc, out = run(cmd)
    assert rc == 0, out[-3000:]
    rc, out = run([str(exe)], env=ENV, timeout=600)
    assert rc == 0 and "0 failure(s)" in out, out[-4000:]


@pytest.mark.skipif(GXX is None, reason="g++ not available")
@pytest.mark.parametrize("san", ["address,undefined", "thread"])
def test_host_twin_under_sanitizers(tmp_path, san):
    exe = tmp_path / "host_twin_driver"
    build_and_run([GXX, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-pthread",
                   f"-fsanitize={san}", "-fno-sanitize-recover=all", f"-I{ROOT / 'include'}",
                   str(DRIVERS / "host_twin_driver.cpp"), str(HOST_SRC), "-o", str(exe)], exe)


@pytest.mark.skipif(not Path(HIPCC).exists(), reason="hipcc not available")
def test_libq4_host_code_under_asan_ubsan(tmp_path):
    from bit_block_quantized_q4_amd.build import COMMON_FLAGS, PER_FILE_FLAGS
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    objs, procs = [], []
    for src in sorted((PKG / "csrc").glob("*.hip")):
        obj = tmp_path / (src.stem + ".o")
        objs.append(obj)
        procs.append(subprocess.Popen([HIPCC, *COMMON_FLAGS, *PER_FILE_FLAGS.get(src.name, []),
                                       *host_san, "-c", str(src), "-o", str(obj)],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, out[-3000:]
    drv = tmp_path / "abi_driver.o"
    rc, out = run([HIPCC, "-std=c++17", *host_san, f"-I{ROOT / 'include'}", "-x", "c++", "-c",
                   str(DRIVERS / "abi_driver.cpp"), "-o", str(drv)])
    assert rc == 0, out[-3000:]
    exe = tmp_path / "abi_driver"
    build_and_run([HIPCC, f"--offload-arch={os.environ.get('Q4_OFFLOAD_ARCH', 'gfx950')}",
                   *host_san, str(drv), *map(str, objs), "-o", str(exe)], exe)
