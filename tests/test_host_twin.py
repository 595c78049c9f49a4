"""The host-CPU twin of the decode GEMV (libq4host, include/q4_host.h) against
the oracle, on the CPU: the same packed bytes as the GPU path, every output
within 1e-3 * sum|w*x| + 1e-6, exact where the arithmetic is exact, and the
same bits whatever the thread count."""

import ctypes
import re
from pathlib import Path

import numpy as np
import pytest

import oracle
import synth
from _golden import load

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "q4_host.h"
BLOCKS, GEMVS = load()
TDT = {"f16": np.float16, "f32": np.float32}
OK, INVALID, SHAPE, DTYPE = 0, 1, 2, 3
F32, F16 = 0, 1


@pytest.fixture(scope="module")
def host():
    from bit_block_quantized_q4_amd import host as h
    if not h.HOST_LIB_PATH.exists():
        from bit_block_quantized_q4_amd.build import build_host
        build_host()
    h.host_lib()
    return h


def assert_close(g, x, packed, n, k, what=""):
    y, S = oracle.matmul_ref(x, packed, n, k)
    ok, worst, idx = oracle.check(g, y, S)
    assert ok, f"{what}: worst |host-oracle|/bound = {worst:.3g} at {idx}"


def test_header_and_exports(host):
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    names = sorted(set(re.findall(r"\b(q4_host_[a-z0-9_]+)\s*\(", text)))
    assert names == sorted(host._SIGS)
    L = ctypes.CDLL(str(host.HOST_LIB_PATH))
    for fn in names:
        assert hasattr(L, fn)
    assert host.host_lib().q4_host_abi_version() == 1
    assert host.q4_host_default_threads() >= 1


def test_golden_worked_dot(host):
    """Hand-worked block A times 32 ones: y = -2.0 exactly."""
    blk = next(b for b in BLOCKS if b.name == "A")
    packed = oracle.quantize(blk.x[None, :])
    for xdt in ("f16", "f32"):
        y = host.q4_host_gemv(np.ones((1, 32), TDT[xdt]), packed)
        assert y[0, 0] == -2.0


@pytest.mark.parametrize("xdt", ["f16", "f32"])
def test_one_hot_rows_give_exact_weights(host, xdt):
    """x = identity: y[i, r] = (q - 8) * d of element i, exactly (pins the
    nibble order on every row, including the rows past the last group of four)."""
    n, k = 71, 96
    w = synth.random_weights(3, n, k, "student_t")
    packed = oracle.quantize(w)
    deq = oracle.dequantize(packed, n, k)
    for r0 in (0, 32, 64):
        x = np.zeros((32, k), TDT[xdt])
        x[np.arange(32), r0 + np.arange(32)] = 1
        y = host.q4_host_gemv(x, packed)
        assert np.array_equal(y, deq[:, r0:r0 + 32].T)


@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8, 16, 17, 31, 32])
@pytest.mark.parametrize("n,k", [(1, 32), (3, 96), (7, 512), (129, 2080), (300, 5120)])
def test_shapes(host, m, n, k):
    w = synth.random_weights(m + n + k, n, k, "outlier")
    x = synth.random_activations(m * 3 + k, m, k, "f16")
    packed = oracle.quantize(w)
    assert_close(host.q4_host_gemv(x, packed, y_dtype=np.float16), x, packed, n, k,
                 what=f"m{m} n{n} k{k}")


@pytest.mark.parametrize("xdt,ydt", [("f32", "f32"), ("f32", "f16"), ("f16", "f32"), ("f16", "f16")])
def test_dtypes(host, xdt, ydt):
    n, k, m = 257, 1056, 13
    w = synth.random_weights(5, n, k, "student_t")
    x = synth.random_activations(6 + m, m, k, xdt)
    packed = oracle.quantize(w)
    assert_close(host.q4_host_gemv(x, packed, y_dtype=TDT[ydt]), x, packed, n, k,
                 what=f"{xdt}->{ydt}")


def test_fp16_output_is_the_rounded_fp32_sum(host):
    n, k, m = 130, 512, 6
    packed = oracle.quantize(synth.random_weights(8, n, k))
    x = synth.random_activations(9, m, k, "f16")
    y32 = host.q4_host_gemv(x, packed, y_dtype=np.float32)
    y16 = host.q4_host_gemv(x, packed, y_dtype=np.float16)
    assert np.array_equal(y16.view(np.uint16), y32.astype(np.float16).view(np.uint16))


def test_edge_case_weights(host):
    """Every quantiser corner case, including scales far above the fp16 weight range."""
    n, k = 96, 32 * 24
    w = synth.edge_case_weights(7, n, k)
    x = synth.random_activations(8, 10, k, "f16")
    packed = oracle.quantize(w)
    assert_close(host.q4_host_gemv(x, packed), x, packed, n, k, what="edge")


def test_same_bits_for_any_thread_count(host):
    n, k, m = 1031, 2048, 10
    packed = oracle.quantize(synth.random_weights(11, n, k, "student_t"))
    x = synth.random_activations(12, m, k, "f16")
    ref = host.q4_host_gemv(x, packed, threads=1)
    for t in (2, 3, 5, 8, 0):
        y = host.q4_host_gemv(x, packed, threads=t)
        assert np.array_equal(y.view(np.uint32), ref.view(np.uint32)), f"threads={t}"
    assert_close(ref, x, packed, n, k, what="threads")


def test_argument_checks(host):
    f = host.host_lib().q4_host_gemv
    x = np.zeros((4, 64), np.float16)
    p = np.zeros(8 * 2 * 18, np.uint8)
    y = np.zeros((4, 8), np.float32)
    X, P, Y = x.ctypes.data, p.ctypes.data, y.ctypes.data
    assert f(X, F16, P, Y, F32, 4, 8, 64, 1) == OK
    assert f(None, F16, P, Y, F32, 4, 8, 64, 1) == INVALID
    assert f(X, F16, None, Y, F32, 4, 8, 64, 1) == INVALID
    assert f(X, F16, P, None, F32, 4, 8, 64, 1) == INVALID
    assert f(X, F16, P, Y, F32, 0, 8, 64, 1) == SHAPE
    assert f(X, F16, P, Y, F32, 33, 8, 64, 1) == SHAPE
    assert f(X, F16, P, Y, F32, 4, 0, 64, 1) == SHAPE
    assert f(X, F16, P, Y, F32, 4, 8, 40, 1) == SHAPE
    assert f(X, F16, P, Y, F32, 4, 8, 0, 1) == SHAPE
    assert f(X, F16, P, Y, F32, 4, 1 << 30, 1 << 20, 1) == SHAPE
    assert f(X, 5, P, Y, F32, 4, 8, 64, 1) == DTYPE
    assert f(X, F16, P, Y, -1, 4, 8, 64, 1) == DTYPE
    assert f(X, F16, P, X, F32, 4, 8, 64, 1) == INVALID      # y overlaps x
    assert f(X, F16, P, P + 16, F32, 1, 8, 64, 1) == INVALID  # y inside packed
    with pytest.raises(host.Q4HostError):
        host.q4_host_gemv(np.zeros((33, 64), np.float16), p, n=8, k=64)
