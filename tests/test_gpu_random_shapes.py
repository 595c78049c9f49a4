"""A seeded sweep of random shapes through the whole path: q4_quantize's bytes
on sampled rows, then q4_gemv (m <= 32) or q4_gemm on sampled output columns,
against the oracle.  Shapes mix random sizes with sizes a few rows either side
of the launch plans' boundaries (multiples of 16 rows per compute unit and of
136 x 16, GEMM row counts near multiples of its 128- and 256-row tiles), K
from 32 up to 17408 on every path's K granularity (512, 256, 64, 32), and
fp16 / bf16 / fp32 activations with fp16 or fp32 outputs.  The case list is
drawn once from a fixed seed, so every run checks the same cases.  A longer
sweep: Q4_RANDOM_CASES=<count> (and Q4_RANDOM_SEED=<seed> for another list)."""

import math
import os

import numpy as np
import pytest

import oracle
import synth
from _gpu import to_dev, to_dev_bf16, to_host

pytestmark = pytest.mark.gpu

N_CASES = int(os.environ.get("Q4_RANDOM_CASES", "48"))
MAX_WEIGHTS = 16_000_000   # n * k, so the host side stays well under a minute in all
MAX_GEMM_XK = 8_000_000    # m * k for the GEMM's activations


def draw_cases(seed=20261202):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(N_CASES):
        op = "gemv" if i % 5 < 3 else "gemm"
        unit = int(rng.choice([512, 256, 64, 32], p=[0.5, 0.2, 0.15, 0.15]))
        if i % 2 == 0:
            k = unit * int(rng.integers(1, 17408 // unit + 1))
            n = int(round(math.exp(rng.uniform(0.0, math.log(60000)))))
            n = max(1, min(n, MAX_WEIGHTS // k))
        else:
            # a plan boundary: n first, then a K the weight budget allows
            step = int(rng.choice([16 * 256, 4 * 256, 2 * 16 * 256, 136 * 16]))
            n = max(1, step * int(rng.integers(1, 9)) + int(rng.integers(-20, 21)))
            n = min(n, MAX_WEIGHTS // unit)
            kmax = max(unit, min(17408, MAX_WEIGHTS // n) // unit * unit)
            k = unit * int(rng.integers(1, kmax // unit + 1))
        if op == "gemv":
            m = int(rng.integers(1, 33))
        else:
            m = int(rng.choice([128, 256])) * int(rng.integers(1, 17)) + int(rng.integers(-3, 4)) \
                if i % 2 else int(round(math.exp(rng.uniform(0.0, math.log(4096)))))
            m = max(1, min(m, MAX_GEMM_XK // k))
        xdt = str(rng.choice(["f16", "f16", "bf16", "f32"]))
        ydt = str(rng.choice(["f16", "f32"]))
        dist = str(rng.choice(["normal", "student_t", "outlier"]))
        cases.append((op, m, n, k, xdt, ydt, dist))
    return cases


CASES = draw_cases(int(os.environ.get("Q4_RANDOM_SEED", "20261202")))


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-m{c[1]}-n{c[2]}-k{c[3]}-{c[4]}-{c[5]}"
                                             for c in CASES])
def test_random_shape_matches_oracle(q4lib, gpu, case):
    op, m, n, k, xdt, ydt, dist = case
    import torch
    seed = (m * 131 + n * 7 + k) % 100003
    w = synth.random_weights(seed, n, k, dist)
    # fp16 outputs: keep |y| well inside fp16's range
    if ydt == "f16":
        w = w * np.float32(0.05)
    packed_d = q4lib.q4_quantize(to_dev(w, gpu))
    packed = to_host(packed_d).reshape(n, -1)
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, size=min(n, 24))]))
    assert np.array_equal(packed[rows], oracle.quantize(w[rows]).reshape(len(rows), -1))

    xa = synth.random_activations(seed + 1, m, k, xdt)
    xd = to_dev_bf16(xa, gpu) if xdt == "bf16" else to_dev(xa, gpu)
    xh = oracle.widen_bf16(xa) if xdt == "bf16" else xa
    ytd = torch.float16 if ydt == "f16" else torch.float32
    if op == "gemv":
        y = q4lib.q4_gemv(xd, packed_d, y_dtype=ytd)
    else:
        y = q4lib.q4_gemm(xd, packed_d, y_dtype=ytd)
    # output columns: first, last, both sides of every multiple of 16 up to
    # 8 x 144, and a random sample, within a host budget of m * cols * k
    budget = int(max(16, min(384, 4e8 / max(1, m * k))))
    cols = {0, n - 1} | {int(c) for c in rng.integers(0, n, size=min(n, budget))}
    for c in range(16, min(n, 8 * 144), 16):
        cols |= {c - 1, c}
    cols = np.array(sorted(cols))
    if len(cols) > 2 * budget:
        keep = np.unique(np.concatenate([[0, len(cols) - 1],
                                         rng.choice(len(cols), size=2 * budget, replace=False)]))
        cols = cols[keep]
    yref, S = oracle.matmul_ref(xh, packed, n, k, cols=cols)
    g = to_host(y[:, torch.from_numpy(cols).to(gpu)].float())
    ok, worst, idx = oracle.check(g, yref, S)
    assert ok, f"worst |gpu-oracle|/bound = {worst:.3g} at {idx}: gpu={g[idx]!r} oracle={yref[idx]!r}"
