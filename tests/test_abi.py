"""C-ABI checks that need no GPU: exports, sizes, status strings and every
host-side argument check (these return before anything is launched)."""

import ctypes
import re
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "q4.h"

OK, INVALID, SHAPE, DTYPE, ALIGN, HIP, WORKSPACE, UNSUPPORTED, SCRATCH = range(9)
F32, F16, BF16 = 0, 1, 2
A = 0x10000          # stand-in, 16-byte aligned "device" addresses: never dereferenced
B = 0x20000000
C = 0x40000000


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q4_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for fn in ["q4_abi_version", "q4_status_string", "q4_packed_size", "q4_quantize",
               "q4_gemv", "q4_gemm_workspace_size", "q4_gemm"]:
        assert fn in names


def test_library_exports_every_declared_symbol(q4lib):
    L = ctypes.CDLL(str(q4lib.LIB_PATH))
    for fn in declared_functions():
        assert hasattr(L, fn), f"{fn} declared in q4.h but not exported"
    assert set(declared_functions()) == set(q4lib._SIGS), "binding and header disagree"


def test_version_and_status_strings(q4lib):
    assert q4lib.q4_abi_version() == 1
    for code in range(9):
        s = q4lib.q4_status_string(code)
        assert s and "unknown" not in s
    assert "unknown" in q4lib.q4_status_string(99)


@pytest.mark.parametrize("n,k,size", [
    (1, 32, 18), (512, 512, 147456), (5120, 5120, 14745600), (17408, 5120, 50135040),
    (1024, 5120, 2949120), (5120, 17408, 50135040), (3, 96, 162),
    (0, 32, 0), (1, 0, 0), (1, 48, 0), (1, 16, 0), (-1, 32, 0)])
def test_packed_size(q4lib, n, k, size):
    assert q4lib.q4_packed_size(n, k) == size


def test_quantize_argument_checks(q4lib):
    f = q4lib.lib().q4_quantize
    assert f(None, F32, 4, 32, B, None) == INVALID
    assert f(A, F32, 4, 32, None, None) == INVALID
    assert f(A, F32, 0, 32, B, None) == SHAPE
    assert f(A, F32, 4, 48, B, None) == SHAPE
    assert f(A, F32, 4, 0, B, None) == SHAPE
    assert f(A, 3, 4, 32, B, None) == DTYPE
    assert f(A + 4, F32, 4, 32, B, None) == ALIGN
    assert f(A, F32, 4, 32, B + 2, None) == ALIGN
    assert f(A, F32, 4, 32, A + 256, None) == INVALID      # packed inside w
    assert f(A, F32, 1 << 30, 1 << 20, B, None) == SHAPE   # n*k beyond 2^40


def test_gemv_argument_checks(q4lib):
    f = q4lib.lib().q4_gemv
    assert f(None, F16, B, C, F16, 1, 8, 32, None) == INVALID
    assert f(A, F16, None, C, F16, 1, 8, 32, None) == INVALID
    assert f(A, F16, B, None, F16, 1, 8, 32, None) == INVALID
    assert f(A, F16, B, C, F16, 0, 8, 32, None) == SHAPE
    assert f(A, F16, B, C, F16, 33, 8, 32, None) == SHAPE    # decode batch is at most 32
    assert f(A, F16, B, C, F16, 1, 0, 32, None) == SHAPE
    assert f(A, F16, B, C, F16, 1, 8, 40, None) == SHAPE
    assert f(A, 5, B, C, F16, 1, 8, 32, None) == DTYPE
    assert f(A, F16, B, C, -1, 1, 8, 32, None) == DTYPE
    assert f(A, F16, B, C, BF16, 1, 8, 32, None) == DTYPE    # outputs are fp32 or fp16
    assert f(A, 3, B, C, F16, 1, 8, 32, None) == DTYPE
    assert f(A + 2, F16, B, C, F16, 1, 8, 32, None) == ALIGN
    assert f(A, F16, B + 8, C, F16, 1, 8, 32, None) == ALIGN
    assert f(A, F16, B, C + 1, F16, 1, 8, 32, None) == ALIGN
    assert f(A, F16, B, A, F16, 1, 8, 32, None) == INVALID   # y aliases x
    assert f(A, F16, B, B + 16, F16, 1, 8, 32, None) == INVALID  # y inside packed


def test_gemm_argument_checks(q4lib):
    f = q4lib.lib().q4_gemm
    assert f(A, 7, B, C, F16, 64, 8, 32, None, 0, None) == DTYPE
    assert f(A, F16, B, C, F16, 0, 8, 32, None, 0, None) == SHAPE
    assert f(A, F16, B, C, F16, 64, 8, 33, None, 0, None) == SHAPE
    assert f(A, F16, B, C, 3, 64, 8, 32, None, 0, None) == DTYPE
    assert f(A + 8, F16, B, C, F16, 64, 8, 32, None, 0, None) == ALIGN
    assert f(A, F16, B, A, F16, 64, 8, 32, None, 0, None) == INVALID
    need = q4lib.q4_gemm_workspace_size(64, 8, 32)
    assert need >= 0
    assert q4lib.q4_gemm_workspace_size(0, 8, 32) == 0
    # bf16 activations are staged as fp16 in the workspace
    needb = q4lib.q4_gemm_workspace_size_dt(64, 8, 32, BF16)
    assert needb >= need + 64 * 32 * 2
    assert q4lib.q4_gemm_workspace_size_dt(64, 8, 32, F16) == need
    assert q4lib.q4_gemm_workspace_size_dt(64, 8, 32, F32) == 0   # the exact route needs none
    assert q4lib.q4_gemm_workspace_size_dt(64, 8, 32, 7) == 0
    assert f(A, BF16, B, C, F16, 64, 8, 32, None, 0, None) == WORKSPACE
    assert f(A, BF16, B, C, F16, 64, 8, 32, 0x60000000, needb - 1, None) == WORKSPACE
    assert f(A, BF16, B, C, F16, 64, 8, 32, 0x60000008, needb, None) == ALIGN
    assert f(A, BF16, B, C, F16, 64, 8, 32, A, needb, None) == INVALID    # workspace over x
    assert f(A, BF16, B, C, BF16, 64, 8, 32, 0x60000000, needb, None) == DTYPE


def test_matmul_k_limit(q4lib):
    """k above 2^24 is refused (32-bit per-lane offsets inside the kernels)."""
    k_ok, k_big = 1 << 24, (1 << 24) + 32
    assert q4lib.lib().q4_gemv(A, F16, B, C, F16, 1, 1, k_big, None) == SHAPE
    assert q4lib.lib().q4_gemm(A, F16, B, C, F16, 1, 1, k_big, None, 0, None) == SHAPE
    assert q4lib.lib().q4_gemm_noalloc(A, F16, B, C, F16, 1, 1, k_big, None) == SHAPE
    assert q4lib.q4_gemm_workspace_size_dt(1, 1, k_big, BF16) == 0
    assert q4lib.q4_gemm_workspace_size_dt(1, 1, k_ok, BF16) >= k_ok * 2
    # the quantiser and the packed size have no such limit
    assert q4lib.q4_packed_size(1, k_big) == (k_big // 32) * 18


def test_gemm_noalloc_argument_checks(q4lib):
    """q4_gemm_noalloc validates like q4_gemm and refuses, before any launch,
    calls whose workspace need exceeds its fixed scratch array."""
    f = q4lib.lib().q4_gemm_noalloc
    assert f(None, F16, B, C, F16, 64, 8, 32, None) == INVALID
    assert f(A, 7, B, C, F16, 64, 8, 32, None) == DTYPE
    assert f(A, F16, B, C, F16, 0, 8, 32, None) == SHAPE
    assert f(A + 8, F16, B, C, F16, 64, 8, 32, None) == ALIGN
    assert f(A, F16, B, A, F16, 64, 8, 32, None) == INVALID
    limit = q4lib.NOALLOC_SCRATCH_BYTES
    m, k = 8192, 8192          # bf16 staging alone is m * k * 2 = 128 MiB
    assert q4lib.q4_gemm_workspace_size_dt(m, 64, k, BF16) > limit
    assert f(0x100000000, BF16, 0x800000000, 0xC00000000, F16, m, 64, k, None) == SCRATCH
    header = HEADER.read_text()
    assert f"#define Q4_NOALLOC_SCRATCH_BYTES ({limit >> 20}u << 20)" in header


def test_read_floor_library_exports_and_checks():
    """libq4floor (the benchmark's plain-read kernel) exports the function its
    header declares and refuses bad arguments before any launch."""
    from bit_block_quantized_q4_amd.build import FLOOR_LIB_PATH
    import bench
    text = re.sub(r"/\*.*?\*/", "", (ROOT / "include" / "q4_read_floor.h").read_text(), flags=re.S)
    assert re.findall(r"\b(q4_[a-z0-9_]+)\s*\(", text) == ["q4_read_floor"]
    assert FLOOR_LIB_PATH.exists()
    L = bench.floor_lib()
    assert L.q4_read_floor(None, 16, A, 1, None) == 1
    assert L.q4_read_floor(A, 16, None, 1, None) == 1
    assert L.q4_read_floor(A + 4, 16, A, 1, None) == 1
    assert L.q4_read_floor(A, 24, A, 1, None) == 1
    assert L.q4_read_floor(A, 16, A, 0, None) == 1


def test_mfma_ceiling_exports_and_checks():
    """libq4floor also exports the matrix-core ceiling its second header
    declares, and refuses bad arguments before any launch."""
    import bench
    text = re.sub(r"/\*.*?\*/", "", (ROOT / "include" / "q4_mfma_ceiling.h").read_text(), flags=re.S)
    assert re.findall(r"\b(q4_[a-z0-9_]+)\s*\(", text) == ["q4_mfma_ceiling"]
    L = bench.floor_lib()
    assert L.q4_mfma_ceiling(1, 8, None, 1, None) == 1
    assert L.q4_mfma_ceiling(1, 8, A, 0, None) == 1
    assert L.q4_mfma_ceiling(1, 0, A, 1, None) == 1
    assert bench.ceiling_flop(256, 4096) == 256 * 8 * 4096 * 8 * 2 * 32 * 32 * 16


def test_trace_build_is_separate(q4lib):
    """libq4trace.so (the measurement build) exports the phase-trace setter;
    libq4.so, the product, does not."""
    from bit_block_quantized_q4_amd.build import TRACE_LIB_PATH
    assert TRACE_LIB_PATH.exists()
    assert hasattr(ctypes.CDLL(str(TRACE_LIB_PATH)), "q4_phase_trace_set")
    assert not hasattr(ctypes.CDLL(str(q4lib.LIB_PATH)), "q4_phase_trace_set")


def test_binding_fails_loudly_without_library(q4lib, monkeypatch, tmp_path):
    monkeypatch.setattr(q4lib, "LIB_PATH", tmp_path / "missing.so")
    monkeypatch.setattr(q4lib, "_LIB", None)
    with pytest.raises(q4lib.Q4LibraryMissing):
        q4lib.q4_packed_size(1, 32)


def test_product_path_never_touches_the_oracle():
    pkg = ROOT / "bit_block_quantized_q4_amd"
    for p in list(pkg.rglob("*.py")) + list(pkg.rglob("*.hip")) + list(pkg.rglob("*.hpp")):
        text = p.read_text()
        assert not re.search(r"^\s*(from|import)\s+oracle\b", text, re.M), p
        assert "oracle/" not in text and "oracle." not in text, p


def test_single_hip_runtime(q4lib):
    """libq4 binds to the HIP runtime torch already loaded (one runtime per process)."""
    import torch  # noqa: F401
    q4lib.lib()
    assert len(q4lib.hip_runtimes_loaded()) <= 1
