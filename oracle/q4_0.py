"""CPU oracle for the Q4_0 block-quantised linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check in ``__graft_entry__``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library (no headers, helpers, tables or pre/post-processing); the only
thing both sides consume is the seeded input generator in ``synth``.

What it computes
----------------
The page "Vertical disaggregation: maximizing throughput on heterogeneous
silicon" (section "Every cycle counts: custom kernels") builds its CPU and GPU
kernels around one shared Q4_0 weight format, lists the kernel stages as
nibble unpack, dot product, scale application and batched decode plus a GPU
path onto matrix cores, and requires the output to be deterministic.  The
page never spells the format out.  This library fixes it as follows (the
usual Q4_0 layout):

* weights are split along K into blocks of 32;
* a block stores one fp16 scale ``d`` (2 bytes, little-endian) followed by 16
  code bytes: byte ``i`` holds the 4-bit code of element ``i`` in its low
  nibble and of element ``i + 16`` in its high nibble (18 bytes per block);
* a weight decodes as ``w = (q - 8) * d``;
* the quantiser takes ``m``, the block element of largest magnitude (the first
  one on a tie), sets ``d = fp16(m / -8)`` and
  ``q = min(15, trunc(x / d + 8.5))``.

Readings where that rule is silent (each one is documented with the design
notes of the repository):

* ``x / d`` divides by the fp16-rounded scale widened back to fp32, using a
  correctly rounded fp32 division, then adds 8.5 in fp32 (round to nearest
  even) -- so the codes are a function of fp32 arithmetic only;
* when ``d`` is +0 or -0 (all-zero block, or a scale below half the smallest
  fp16 subnormal) every code is 8;
* fp32 -> fp16 rounds to nearest even, keeps subnormals;
* inputs must be finite and ``|w| < 65520 * 8`` so that ``d`` is finite.

The matmul oracle is the plain definition ``y = x . dequant(W)^T`` evaluated
in fp64 (every product of an fp16/fp32 activation and a dequantised weight is
exact in fp64), together with ``S = sum |x * w|`` which scales the acceptance
bound ``|gpu - y| <= 1e-3 * S + 1e-6``.

bf16 inputs (weights or activations) enter through ``widen_bf16``, the exact
widening of a bfloat16 pattern to binary32; everything after it is unchanged.

Pins (in ``tests/test_oracle.py``): hand-worked blocks derived from the rule
above (``tests/golden``), the round-trip bound ``|x - dequant| <= |d|/2`` on
unclamped elements, code-range and maximum-element invariants, one-hot and
all-ones activations, exact rational brute-force dot products (fp16, fp32
and bf16 activations), and the bf16 widening against a field-by-field
decoding of all 65536 patterns.
"""

from __future__ import annotations

import numpy as np

QK = 32               # weights per block
BLOCK_BYTES = 18      # 2-byte fp16 scale + 16 code bytes
CODE_BYTES = 16


def packed_size(n: int, k: int) -> int:
    """Bytes of a packed [n, k] weight: n rows of k/32 consecutive 18-byte blocks."""
    if k % QK:
        raise ValueError("k must be a multiple of 32")
    return n * (k // QK) * BLOCK_BYTES


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> the values they denote, as fp32.

    A bfloat16 value is the upper half of an IEEE binary32 pattern (sign, the
    8-bit exponent, the top 7 fraction bits), so appending 16 zero bits gives
    the same value in binary32 exactly.  bf16 weights and activations enter
    the oracle through this widening; the quantiser and matmul definitions
    below then apply unchanged.
    """
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        raise TypeError(f"bf16 patterns must be uint16, got {b.dtype}")
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _as_f32(w: np.ndarray) -> np.ndarray:
    """fp16 widens to fp32 exactly; fp32 passes through."""
    if w.dtype == np.float16:
        return w.astype(np.float32)
    if w.dtype == np.float32:
        return w
    raise TypeError(f"unsupported weight dtype {w.dtype}")


def quantize(w: np.ndarray) -> np.ndarray:
    """Q4_0-encode a row-major [n, k] fp32/fp16 weight into [n, k/32*18] bytes.

    Steps, per block of 32 along K (section "Every cycle counts: custom
    kernels" of the vertical-disaggregation page requires one format on every
    backend; the arithmetic is the rule stated in the module docstring):

    1. m  = the element of largest |x|; the first index wins a tie
       (np.argmax returns the first maximum).
    2. d  = fp16(m / -8)   (fp32 quotient, rounded to nearest-even fp16).
    3. D  = d widened to fp32 (exact).
    4. q  = min(15, trunc(x / D + 8.5)) with fp32 division and addition;
       q = 8 for every element when D is zero.
    5. pack: bytes 0-1 = d little-endian, byte 2+i = q[i] | q[i+16] << 4.
    """
    x = _as_f32(np.asarray(w))
    if x.ndim != 2 or x.shape[1] % QK:
        raise ValueError("weight must be [n, k] with k a multiple of 32")
    if not np.all(np.isfinite(x)):
        raise ValueError("weights must be finite")
    n, k = x.shape
    nb = k // QK
    xb = x.reshape(n, nb, QK)

    # 1. signed element of largest magnitude, first index on ties
    j = np.argmax(np.abs(xb), axis=-1)
    m = np.take_along_axis(xb, j[..., None], axis=-1)[..., 0]

    # 2-3. fp16 scale and its exact fp32 widening
    t = m / np.float32(-8.0)
    d = t.astype(np.float16)
    if not np.all(np.isfinite(d)):
        raise ValueError("block scale overflows fp16: |w| must stay below 65520*8")
    D = d.astype(np.float32)

    # 4. codes
    zero = (D == 0)
    Dsafe = np.where(zero, np.float32(1.0), D)[..., None]
    u = xb / Dsafe                              # fp32, correctly rounded
    v = u + np.float32(8.5)                     # fp32, round to nearest even
    q = np.minimum(np.float32(15.0), np.trunc(v))
    q = np.maximum(np.float32(0.0), q).astype(np.uint8)
    q[zero] = 8

    # 5. packing
    codes = (q[..., :16] | (q[..., 16:] << 4)).astype(np.uint8)
    dbytes = d.astype("<f2").view(np.uint8).reshape(n, nb, 2)
    blocks = np.concatenate([dbytes, codes], axis=-1)
    return np.ascontiguousarray(blocks.reshape(n, nb * BLOCK_BYTES))


def unpack(packed: np.ndarray, n: int, k: int):
    """Split packed bytes into (d: fp16 [n, k/32], q: uint8 codes [n, k])."""
    nb = k // QK
    blocks = np.asarray(packed, dtype=np.uint8).reshape(n, nb, BLOCK_BYTES)
    d = np.ascontiguousarray(blocks[..., :2]).view("<f2")[..., 0]
    cb = blocks[..., 2:]
    q = np.concatenate([cb & 0x0F, cb >> 4], axis=-1)  # element i, then i+16
    return d, q.reshape(n, k)


def dequantize(packed: np.ndarray, n: int, k: int) -> np.ndarray:
    """w = (q - 8) * d, exact in fp32 (4-bit integer times an 11-bit significand)."""
    d, q = unpack(packed, n, k)
    D = d.astype(np.float32)
    qm8 = q.astype(np.float32).reshape(n, k // QK, QK) - np.float32(8.0)
    return (qm8 * D[..., None]).reshape(n, k)


def matmul_ref(x: np.ndarray, packed: np.ndarray, n: int, k: int, cols=None):
    """(y, S) for y = x . dequant(W)^T and S = |x| . |dequant(W)|^T, both fp64.

    x is a row-major [m, k] fp16/fp32 activation; every product x*w is exact
    in fp64, so y differs from the exact sum only by fp64 summation error.
    ``cols`` optionally restricts the output features to those rows of W
    (y then has len(cols) columns, in that order).
    """
    if cols is not None:
        cols = np.asarray(cols)
        packed = np.asarray(packed).reshape(n, -1)[cols]
        n = len(cols)
    xa = np.asarray(x)
    if xa.dtype not in (np.float16, np.float32):
        raise TypeError(f"unsupported activation dtype {xa.dtype}")
    x64 = xa.astype(np.float64)
    w64 = dequantize(packed, n, k).astype(np.float64)
    y = x64 @ w64.T
    s = np.abs(x64) @ np.abs(w64).T
    return y, s


TOL_REL = 1e-3
TOL_ABS = 1e-6


def tolerance(S: np.ndarray) -> np.ndarray:
    """Acceptance bound on |gpu - y|: 1e-3 * sum|w*x| + 1e-6."""
    return TOL_REL * S + TOL_ABS


def check(g: np.ndarray, y: np.ndarray, S: np.ndarray):
    """Return (ok, worst ratio |g-y|/bound, index of the worst element)."""
    g64 = np.asarray(g).astype(np.float64)
    err = np.abs(g64 - y)
    ratio = err / tolerance(S)
    bad = ~np.isfinite(g64)
    ratio = np.where(bad, np.inf, ratio)
    idx = np.unravel_index(np.argmax(ratio), ratio.shape) if ratio.size else ()
    worst = float(ratio[idx]) if ratio.size else 0.0
    return bool(np.all(ratio <= 1.0)), worst, idx
