"""Seeded synthetic workloads for Q4_0 linears.

The source pages run a 27B-class dense decoder whose weights are stored as
Q4_0 ("Vertical disaggregation: maximizing throughput on heterogeneous
silicon", sections "awkward middle ground" and "results").  No trained weights
or datasets exist here, so every tensor is drawn from a seeded NumPy
generator with the shapes of that model's linears:

* Workload 1 -- one 512 x 512 linear, weights N(0, 0.02) fp32, one fp32
  activation row, fp32 output.
* Workload 2 -- the 5120 x 5120 attention projection in batched decode,
  M in {1, 4, 10, 16}, fp16 activations N(0, 1), fp16 output.
* Workload 3 -- the 17408 x 5120 FFN gate/up projection in batched decode,
  M in {1, 10, 32}; 0.1 % of the Q4_0 blocks (chosen uniformly without
  replacement) scaled x20 before quantisation to create outlier blocks.
* Workload 4 -- the same 17408 x 5120 weight in prefill, 2048 rows of
  activations, run as 8 chunks of 256 rows (the chunk size the chunked-prefill
  page settles on) and as one 2048-row batch.
* Workload 5 -- all seven linears of one decoder layer (q, k, v, o, gate, up,
  down) with heavy-tailed Student-t(nu=3) x 0.02 weights, M in
  {1, 10, 256, 4096}.

Every generator is ``numpy.random.default_rng(SeedSequence([seed, workload,
tensor]))``, so each tensor is reproducible on its own.  Activations for a
workload are drawn once at the largest M and the first M rows are used for
smaller M.
"""

from __future__ import annotations

import hashlib
from dataclasses import dataclass, field
from typing import Dict, List, Sequence, Tuple

import numpy as np

QK = 32  # weights per Q4_0 block along K


@dataclass(frozen=True)
class Linear:
    name: str
    n: int          # output features (rows of W)
    k: int          # input features (columns of W, the quantised axis)
    tensor_id: int  # seed component for this weight


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    linears: Tuple[Linear, ...]
    ms: Tuple[int, ...]
    x_dtype: str          # "f32" or "f16"
    y_dtype: str          # "f32" or "f16"
    dist: str             # "normal", "outlier", "student_t"
    kernel: str           # "gemv", "gemm" or "both"
    chunk: int = 0        # prefill chunk rows (0: no chunking)
    notes: str = ""


_L_ATTN = (
    Linear("q", 5120, 5120, 0),
    Linear("k", 1024, 5120, 1),
    Linear("v", 1024, 5120, 2),
    Linear("o", 5120, 5120, 3),
    Linear("gate", 17408, 5120, 4),
    Linear("up", 17408, 5120, 5),
    Linear("down", 5120, 17408, 6),
)

WORKLOADS: Dict[int, Workload] = {
    1: Workload(1, "single_linear_512", (Linear("w", 512, 512, 0),), (1,),
                "f32", "f32", "normal", "gemv"),
    2: Workload(2, "decode_attn_proj_5120x5120", (Linear("q", 5120, 5120, 0),),
                (1, 4, 10, 16), "f16", "f16", "normal", "gemv"),
    3: Workload(3, "decode_ffn_gate_up_17408x5120_outliers",
                (Linear("gate", 17408, 5120, 0),), (1, 10, 32),
                "f16", "f16", "outlier", "gemv"),
    4: Workload(4, "prefill_chunked_2048x17408x5120",
                (Linear("gate", 17408, 5120, 0),), (2048,),
                "f16", "f16", "normal", "gemm", chunk=256),
    5: Workload(5, "layer_27b_dense_7_linears", _L_ATTN, (1, 10, 256, 4096),
                "f16", "f16", "student_t", "both"),
}

ACT_TENSOR_BASE = 100  # activations use tensor ids 100 + index of their K


def rng_for(seed: int, workload: int, tensor: int) -> np.random.Generator:
    """Independent generator for one tensor of one workload."""
    return np.random.default_rng(np.random.SeedSequence([seed, workload, tensor]))


def normal_weights(rng: np.random.Generator, n: int, k: int,
                   sigma: float = 0.02) -> np.ndarray:
    w = rng.standard_normal((n, k), dtype=np.float32)
    w *= np.float32(sigma)
    return w


def outlier_weights(rng: np.random.Generator, n: int, k: int,
                    sigma: float = 0.02, frac: float = 0.001,
                    scale: float = 20.0) -> np.ndarray:
    """N(0, sigma) weights with round(frac * blocks) whole 32-wide blocks x scale."""
    w = normal_weights(rng, n, k, sigma)
    nblocks = n * (k // QK)
    count = int(round(frac * nblocks))
    pick = rng.choice(nblocks, size=count, replace=False)
    wb = w.reshape(nblocks, QK)
    wb[pick] *= np.float32(scale)
    return w


def student_t_weights(rng: np.random.Generator, n: int, k: int,
                      sigma: float = 0.02) -> np.ndarray:
    """Student-t with 3 degrees of freedom, times sigma.

    Drawn from the definition t = Z / sqrt(V / 3) with V ~ chi-square(3),
    and V built as chi-square(2) + chi-square(1) = -2 ln U + Z1^2
    (U uniform on (0, 1], Z, Z1 standard normal, all independent).
    """
    w = rng.standard_normal((n, k), dtype=np.float32)
    v = rng.standard_normal((n, k), dtype=np.float32)
    np.multiply(v, v, out=v)
    u = rng.random((n, k), dtype=np.float32)
    np.subtract(np.float32(1.0), u, out=u)          # (0, 1]
    np.log(u, out=u)
    v -= np.float32(2.0) * u
    del u
    v *= np.float32(1.0 / 3.0)
    np.sqrt(v, out=v)
    w /= v
    w *= np.float32(sigma)
    return w


def workload_weights(wl: Workload, lin: Linear, seed: int = 0) -> np.ndarray:
    rng = rng_for(seed, wl.wid, lin.tensor_id)
    if wl.dist == "normal":
        return normal_weights(rng, lin.n, lin.k)
    if wl.dist == "outlier":
        return outlier_weights(rng, lin.n, lin.k)
    if wl.dist == "student_t":
        return student_t_weights(rng, lin.n, lin.k)
    raise ValueError(wl.dist)


def workload_activations(wl: Workload, k: int, m: int, seed: int = 0) -> np.ndarray:
    """First m rows of the workload's activation draw for input width k."""
    ks = sorted({lin.k for lin in wl.linears})
    rng = rng_for(seed, wl.wid, ACT_TENSOR_BASE + ks.index(k))
    mmax = max(wl.ms)
    if m > mmax:
        raise ValueError(f"m={m} exceeds the workload's largest batch {mmax}")
    x = rng.standard_normal((mmax, k), dtype=np.float32)[:m]
    if wl.x_dtype == "f16":
        return np.ascontiguousarray(x.astype(np.float16))
    return np.ascontiguousarray(x)


# ---------------------------------------------------------------- small cases

def random_weights(seed: int, n: int, k: int, dist: str = "normal") -> np.ndarray:
    """Weights for shape sweeps (workload id 0 marks 'not a named workload')."""
    rng = rng_for(seed, 0, 1 + n * 7 + k * 13)
    if dist == "normal":
        return normal_weights(rng, n, k)
    if dist == "outlier":
        return outlier_weights(rng, n, k, frac=0.05)
    if dist == "student_t":
        return student_t_weights(rng, n, k)
    raise ValueError(dist)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 draws rounded to bfloat16 (nearest even), as uint16 bit patterns:
    how bf16 inputs are made from the fp32 draws (finite values only)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def random_activations(seed: int, m: int, k: int, dtype: str = "f16") -> np.ndarray:
    """N(0, 1) activations: fp32, rounded to fp16, or rounded to bf16 and
    returned as uint16 bit patterns ("bf16")."""
    rng = rng_for(seed, 0, 2 + m * 11 + k * 17)
    x = rng.standard_normal((m, k), dtype=np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(x.astype(np.float16))
    if dtype == "bf16":
        return bf16_bits(x)
    return x


def edge_case_weights(seed: int, n: int, k: int, top: float = 5.0e5) -> np.ndarray:
    """Rows of Q4_0 blocks that exercise every corner of the quantiser rule.

    Each 32-wide block gets one pattern, cycling through: ordinary N(0,1)
    scaled values; all +0; all -0; +a/-a magnitude ties (first index must
    win); a constant block; values small enough that the fp16 scale is
    subnormal or rounds to zero; values near the top of the fp16 scale
    range (magnitudes up to ``top``); one huge element among tiny ones; exact
    multiples of the scale (ties at the rounding boundary); and blocks whose
    maximum sits at the last index.
    """
    rng = rng_for(seed, 0, 3 + n * 19 + k * 23)
    nb = k // QK
    out = np.empty((n, nb, QK), dtype=np.float32)
    patterns = 12
    for r in range(n):
        for b in range(nb):
            p = (r * nb + b) % patterns
            v = rng.standard_normal(QK).astype(np.float32)
            if p == 0:
                blk = v * np.float32(0.02)
            elif p == 1:
                blk = np.zeros(QK, np.float32)
            elif p == 2:
                blk = np.full(QK, -0.0, np.float32)
            elif p == 3:
                a = np.float32(abs(v[0]) + 0.5)
                blk = v * np.float32(0.1)
                i, j = sorted(rng.choice(QK, 2, replace=False))
                blk[i], blk[j] = (a, -a) if rng.random() < 0.5 else (-a, a)
            elif p == 4:
                blk = np.full(QK, np.float32(rng.choice([-1, 1]) * abs(v[1]) + 0.01))
            elif p == 5:
                blk = v * np.float32(1e-6)        # d lands in fp16 subnormals
            elif p == 6:
                blk = v * np.float32(1e-9)        # d rounds to (signed) zero
            elif p == 7:
                blk = v * np.float32(top / 12.0)  # d near the top of its range
                blk = np.clip(blk, -top, top).astype(np.float32)
            elif p == 8:
                blk = v * np.float32(1e-4)
                blk[rng.integers(QK)] = np.float32(rng.choice([-1, 1]) * 3.0)
            elif p == 9:
                d = np.float32(rng.choice([0.25, 0.125, 0.0625]))
                blk = (rng.integers(-8, 8, QK).astype(np.float32) + np.float32(0.5)) * d
                blk[0] = -8 * d                   # pins the scale exactly
            elif p == 10:
                blk = v * np.float32(0.05)
                blk[-1] = np.float32(np.sign(v[-1]) or 1.0) * (np.abs(blk).max() + 0.01)
            else:
                blk = (v * np.float32(0.02)).astype(np.float16).astype(np.float32)
            out[r, b] = blk
    return out.reshape(n, k)


def sha256_of(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]
