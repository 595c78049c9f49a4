"""Binding of libq4host (``include/q4_host.h``): the host-CPU twin of
``q4_gemv`` over the same packed Q4_0 bytes, for numpy arrays in host memory.

A separate backend, chosen explicitly by the caller: the GPU binding never
calls it.  If ``libq4host.so`` is not built every call raises
``Q4LibraryMissing`` (build it with ``python -m bit_block_quantized_q4_amd.build``).
"""

from __future__ import annotations

import ctypes
from typing import Optional

import numpy as np

from . import BLOCK_BYTES, GEMV_MAX_M, PKG_DIR, QK, Q4_F16, Q4_F32, Q4_OK, Q4LibraryMissing

HOST_LIB_PATH = PKG_DIR / "libq4host.so"
HOST_ABI_VERSION = 1
Q4_ERR_UNSUPPORTED = 7

_SIGS = {
    "q4_host_abi_version": (ctypes.c_int, []),
    "q4_host_default_threads": (ctypes.c_int, []),
    "q4_host_gemv": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_int64, ctypes.c_int]),
}

_STATUS = {
    1: "invalid argument (null pointer or overlapping buffers)",
    2: "invalid shape (need 1 <= m <= 32, n >= 1, k >= 32, k % 32 == 0)",
    3: "unsupported dtype",
    Q4_ERR_UNSUPPORTED: "the host CPU lacks AVX2, FMA or F16C",
}

_HLIB: Optional[ctypes.CDLL] = None


class Q4HostError(RuntimeError):
    """A libq4host call returned a non-OK status."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({_STATUS.get(status, 'unknown status')})")


def host_lib() -> ctypes.CDLL:
    """The loaded libq4host.so (raises Q4LibraryMissing when absent)."""
    global _HLIB
    if _HLIB is None:
        if not HOST_LIB_PATH.exists():
            raise Q4LibraryMissing(
                f"{HOST_LIB_PATH} is not built; run `python -m bit_block_quantized_q4_amd.build`")
        try:
            L = ctypes.CDLL(str(HOST_LIB_PATH))
        except OSError as e:  # pragma: no cover - depends on the host
            raise Q4LibraryMissing(f"cannot load {HOST_LIB_PATH}: {e}") from e
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        if L.q4_host_abi_version() != HOST_ABI_VERSION:
            raise Q4LibraryMissing("libq4host.so ABI version mismatch; rebuild it")
        _HLIB = L
    return _HLIB


def q4_host_default_threads() -> int:
    return host_lib().q4_host_default_threads()


def _code(a: np.ndarray, what: str) -> int:
    if a.dtype == np.float32:
        return Q4_F32
    if a.dtype == np.float16:
        return Q4_F16
    raise TypeError(f"{what} must be float32 or float16, got {a.dtype}")


def q4_host_gemv(x: np.ndarray, packed: np.ndarray, y: Optional[np.ndarray] = None,
                 y_dtype=np.float32, n: Optional[int] = None, k: Optional[int] = None,
                 threads: int = 0) -> np.ndarray:
    """Host batched-decode GEMV y[m, n] = x[m, k] . dequant(W)^T, 1 <= m <= 32,
    on the packed bytes q4_quantize writes (a [n, k/32*18] uint8 array, or a
    flat one with n and k given)."""
    x = np.ascontiguousarray(x)
    packed = np.ascontiguousarray(packed)
    if packed.dtype != np.uint8:
        raise TypeError("packed must be uint8")
    if n is None or k is None:
        if packed.ndim != 2 or packed.shape[1] % BLOCK_BYTES != 0:
            raise ValueError("packed must be [n, k/32*18] unless n and k are given")
        n, k = packed.shape[0], packed.shape[1] // BLOCK_BYTES * QK
    if x.ndim == 1:
        x = x.reshape(1, -1)
    m = int(x.shape[0])
    if x.ndim != 2 or x.shape[1] != k:
        raise ValueError(f"x must be [m, {k}]")
    if packed.size != n * (k // QK) * BLOCK_BYTES:
        raise ValueError("packed has the wrong size for n and k")
    if y is None:
        y = np.empty((m, n), dtype=y_dtype)
    if not (y.flags.c_contiguous and y.shape == (m, n)):
        raise ValueError(f"y must be a contiguous [{m}, {n}] array")
    st = host_lib().q4_host_gemv(x.ctypes.data, _code(x, "x"), packed.ctypes.data,
                                 y.ctypes.data, _code(y, "y"), m, n, k, int(threads))
    if st != Q4_OK:
        raise Q4HostError(st, "q4_host_gemv")
    return y


__all__ = ["HOST_LIB_PATH", "host_lib", "q4_host_default_threads", "q4_host_gemv",
           "Q4HostError", "Q4_ERR_UNSUPPORTED", "GEMV_MAX_M"]
