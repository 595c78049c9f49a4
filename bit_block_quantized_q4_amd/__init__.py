"""libq4: Q4_0 block-quantised linear layers on AMD MI355X (gfx950).

This module is the thin Python binding over the C ABI declared in
``include/q4.h``: it marshals torch device tensors into pointers, dtype codes
and a HIP stream handle and calls ``libq4.so``.  Every step of the
computation runs in the library's HIP kernels; there is no fallback.  If the
library has not been built, every call raises ``Q4LibraryMissing`` (build it
with ``python -m bit_block_quantized_q4_amd.build``).

Functions mirror the C entry points: ``q4_packed_size``,
``q4_gemm_workspace_size``, ``q4_gemm_workspace_size_dt``, ``q4_quantize``, ``q4_gemv``, ``q4_gemm``,
``q4_gemm_noalloc``, ``q4_status_string``, ``q4_abi_version``.
"""

from __future__ import annotations

import ctypes
from pathlib import Path
from typing import Optional, Tuple

PKG_DIR = Path(__file__).resolve().parent
LIB_PATH = PKG_DIR / "libq4.so"
HEADER_PATH = PKG_DIR.parent / "include" / "q4.h"

ABI_VERSION = 1
QK = 32
BLOCK_BYTES = 18
GEMV_MAX_M = 32

Q4_OK = 0
Q4_ERR_INVALID_ARG = 1
Q4_ERR_SHAPE = 2
Q4_ERR_DTYPE = 3
Q4_ERR_ALIGNMENT = 4
Q4_ERR_HIP = 5
Q4_ERR_WORKSPACE = 6
Q4_ERR_UNSUPPORTED = 7
Q4_ERR_SCRATCH = 8
NOALLOC_SCRATCH_BYTES = 64 << 20

Q4_F32 = 0
Q4_F16 = 1
Q4_BF16 = 2

# Every function the header declares, with (restype, argtypes).
_SIGS = {
    "q4_abi_version": (ctypes.c_int, []),
    "q4_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "q4_packed_size": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64]),
    "q4_gemm_workspace_size": (ctypes.c_size_t, [ctypes.c_int64] * 3),
    "q4_gemm_workspace_size_dt": (ctypes.c_size_t, [ctypes.c_int64] * 3 + [ctypes.c_int]),
    "q4_quantize": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                   ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]),
    "q4_gemv": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                               ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                               ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]),
    "q4_gemm": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                               ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                               ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                               ctypes.c_size_t, ctypes.c_void_p]),
    "q4_gemm_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]),
}


class Q4LibraryMissing(RuntimeError):
    """libq4.so is not built or cannot be loaded."""


class Q4Error(RuntimeError):
    """A libq4 call returned a non-OK status."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({q4_status_string(status)})")


_LIB: Optional[ctypes.CDLL] = None


def hip_runtimes_loaded():
    """Distinct libamdhip64 files mapped into this process (Linux)."""
    try:
        maps = Path("/proc/self/maps").read_text()
    except OSError:  # pragma: no cover
        return []
    return sorted({ln.split()[-1] for ln in maps.splitlines()
                   if "libamdhip64" in ln and ln.split()[-1].startswith("/")})


def lib() -> ctypes.CDLL:
    """The loaded libq4.so (raises Q4LibraryMissing when absent)."""
    global _LIB
    if _LIB is None:
        if not LIB_PATH.exists():
            raise Q4LibraryMissing(
                f"{LIB_PATH} is not built; run `python -m bit_block_quantized_q4_amd.build`")
        # torch ships its own HIP runtime under the same soname as ROCm's.  Load
        # torch first so libq4 binds to that runtime: device pointers and streams
        # handed over by torch are only valid inside the runtime that made them.
        try:
            import torch  # noqa: F401
        except ImportError:  # pragma: no cover - a C caller without torch
            pass
        try:
            L = ctypes.CDLL(str(LIB_PATH))
        except OSError as e:  # pragma: no cover - depends on the host
            raise Q4LibraryMissing(f"cannot load {LIB_PATH}: {e}") from e
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        if L.q4_abi_version() != ABI_VERSION:
            raise Q4LibraryMissing("libq4.so ABI version mismatch; rebuild it")
        runtimes = hip_runtimes_loaded()
        if len(runtimes) > 1:
            raise Q4LibraryMissing(
                "two HIP runtimes are loaded in this process (" + ", ".join(runtimes) +
                "); import torch before loading libq4")
        _LIB = L
    return _LIB


# ------------------------------------------------------------ plain wrappers

def q4_abi_version() -> int:
    return lib().q4_abi_version()


def q4_status_string(status: int) -> str:
    return lib().q4_status_string(int(status)).decode()


def q4_packed_size(n: int, k: int) -> int:
    return lib().q4_packed_size(int(n), int(k))


def q4_gemm_workspace_size(m: int, n: int, k: int) -> int:
    return lib().q4_gemm_workspace_size(int(m), int(n), int(k))


def q4_gemm_workspace_size_dt(m: int, n: int, k: int, x_dtype: int) -> int:
    return lib().q4_gemm_workspace_size_dt(int(m), int(n), int(k), int(x_dtype))


# ------------------------------------------------------------ torch marshalling

def _torch():
    import torch  # imported lazily: the symbol checks above need no torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return Q4_F32
    if t.dtype == torch.float16:
        return Q4_F16
    if t.dtype == torch.bfloat16:
        return Q4_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; libq4 takes float32, float16 or bfloat16")


def _torch_dtype(code_or_dtype):
    torch = _torch()
    if code_or_dtype in (Q4_F32, torch.float32, "f32", "float32"):
        return torch.float32
    if code_or_dtype in (Q4_F16, torch.float16, "f16", "float16"):
        return torch.float16
    raise TypeError(f"unsupported output dtype {code_or_dtype!r}")


def _stream_handle(stream, device) -> int:
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _need_device(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def packed_shape(packed, n: Optional[int] = None, k: Optional[int] = None) -> Tuple[int, int]:
    """(n, k) of a packed weight: [n, k/32*18] uint8 unless given explicitly."""
    if n is not None and k is not None:
        return int(n), int(k)
    if packed.dim() != 2 or packed.shape[1] % BLOCK_BYTES:
        raise ValueError("packed must be [n, k/32*18] uint8, or pass n and k")
    return int(packed.shape[0]), int(packed.shape[1] // BLOCK_BYTES * QK)


def _check(status: int, what: str):
    if status != Q4_OK:
        raise Q4Error(status, what)


def q4_quantize(w, packed=None, stream=None):
    """Quantise a [n, k] fp32/fp16/bf16 device weight into a [n, k/32*18] uint8 tensor."""
    torch = _torch()
    _need_device(w, "w")
    if w.dim() != 2:
        raise ValueError("w must be 2-D [n, k]")
    n, k = int(w.shape[0]), int(w.shape[1])
    if packed is None:
        packed = torch.empty((n, (k // QK) * BLOCK_BYTES), dtype=torch.uint8, device=w.device)
    _need_device(packed, "packed")
    _check(lib().q4_quantize(w.data_ptr(), _dtype_code(w), n, k, packed.data_ptr(),
                             _stream_handle(stream, w.device)), "q4_quantize")
    return packed


def _out(x, m, n, y, y_dtype):
    torch = _torch()
    if y is None:
        # outputs are fp32 or fp16: bf16 activations default to an fp32 output
        dflt = torch.float32 if x.dtype == torch.bfloat16 else x.dtype
        y = torch.empty((m, n), dtype=_torch_dtype(y_dtype if y_dtype is not None else dflt),
                        device=x.device)
    _need_device(y, "y")
    return y


def q4_gemv(x, packed, y=None, y_dtype=None, stream=None, n=None, k=None):
    """Batched-decode GEMV y[m, n] = x[m, k] . dequant(W)^T, 1 <= m <= 32."""
    _need_device(x, "x")
    _need_device(packed, "packed")
    n, k = packed_shape(packed, n, k)
    m = int(x.numel() // k) if x.dim() != 2 else int(x.shape[0])
    y = _out(x, m, n, y, y_dtype)
    _check(lib().q4_gemv(x.data_ptr(), _dtype_code(x), packed.data_ptr(), y.data_ptr(),
                         _dtype_code(y), m, n, k, _stream_handle(stream, x.device)), "q4_gemv")
    return y


def q4_gemm(x, packed, y=None, y_dtype=None, workspace=None, stream=None, n=None, k=None):
    """Prefill GEMM y[m, n] = x[m, k] . dequant(W)^T on fp16 MFMA (x fp16, or bf16
    staged as fp16 in the workspace)."""
    torch = _torch()
    _need_device(x, "x")
    _need_device(packed, "packed")
    n, k = packed_shape(packed, n, k)
    m = int(x.numel() // k) if x.dim() != 2 else int(x.shape[0])
    y = _out(x, m, n, y, y_dtype)
    need = q4_gemm_workspace_size_dt(m, n, k, _dtype_code(x))
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wptr = workspace.data_ptr() if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().q4_gemm(x.data_ptr(), _dtype_code(x), packed.data_ptr(), y.data_ptr(),
                         _dtype_code(y), m, n, k, wptr, wbytes,
                         _stream_handle(stream, x.device)), "q4_gemm")
    return y


def q4_gemm_noalloc(x, packed, y, stream=None, n=None, k=None):
    """q4_gemm with its workspace taken from the library's fixed per-device
    scratch array (no allocation by the library; y must be given).  Calls that
    may overlap on one device race on that array."""
    _need_device(x, "x")
    _need_device(packed, "packed")
    _need_device(y, "y")
    n, k = packed_shape(packed, n, k)
    m = int(x.numel() // k) if x.dim() != 2 else int(x.shape[0])
    _check(lib().q4_gemm_noalloc(x.data_ptr(), _dtype_code(x), packed.data_ptr(), y.data_ptr(),
                                 _dtype_code(y), m, n, k, _stream_handle(stream, x.device)),
           "q4_gemm_noalloc")
    return y
