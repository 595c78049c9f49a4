"""The seeded generator: reproducible, right shapes and distributions."""

import numpy as np
from scipy import stats

import synth


def test_workloads_table():
    assert [w.wid for w in synth.WORKLOADS.values()] == [1, 2, 3, 4, 5]
    layer = synth.WORKLOADS[5]
    assert [(l.name, l.n, l.k) for l in layer.linears] == [
        ("q", 5120, 5120), ("k", 1024, 5120), ("v", 1024, 5120), ("o", 5120, 5120),
        ("gate", 17408, 5120), ("up", 17408, 5120), ("down", 5120, 17408)]
    assert synth.WORKLOADS[2].ms == (1, 4, 10, 16)
    assert synth.WORKLOADS[3].ms == (1, 10, 32)


def test_reproducible():
    a = synth.random_weights(3, 8, 64, "student_t")
    b = synth.random_weights(3, 8, 64, "student_t")
    assert synth.sha256_of(a) == synth.sha256_of(b)
    assert not np.array_equal(a, synth.random_weights(4, 8, 64, "student_t"))
    wl = synth.WORKLOADS[1]
    w = synth.workload_weights(wl, wl.linears[0])
    assert w.shape == (512, 512) and w.dtype == np.float32
    assert np.array_equal(w, synth.workload_weights(wl, wl.linears[0]))


def test_activation_prefix_rows():
    wl = synth.WORKLOADS[2]
    x16 = synth.workload_activations(wl, 5120, 16)
    x4 = synth.workload_activations(wl, 5120, 4)
    assert x16.dtype == np.float16 and np.array_equal(x16[:4], x4)
    assert synth.workload_activations(synth.WORKLOADS[1], 512, 1).dtype == np.float32


def test_outlier_blocks():
    rng = synth.rng_for(0, 99, 0)
    w = synth.outlier_weights(rng, 64, 512, frac=0.01)
    blockmax = np.abs(w.reshape(-1, 32)).max(axis=1)
    assert (blockmax > 0.2).sum() == round(0.01 * 64 * 16)


def test_student_t_distribution():
    rng = synth.rng_for(0, 98, 0)
    w = synth.student_t_weights(rng, 64, 4096) / np.float32(0.02)
    assert stats.kstest(w.ravel().astype(np.float64), stats.t(3).cdf).pvalue > 1e-3


def test_normal_distribution():
    rng = synth.rng_for(0, 97, 0)
    w = synth.normal_weights(rng, 64, 4096) / np.float32(0.02)
    assert stats.kstest(w.ravel().astype(np.float64), stats.norm.cdf).pvalue > 1e-3


def test_edge_cases_cover_every_pattern():
    w = synth.edge_case_weights(0, 4, 32 * 12)
    blocks = w.reshape(-1, 32)
    assert np.all(blocks[1] == 0) and not np.any(np.signbit(blocks[1]))
    assert np.all(blocks[2] == 0) and np.all(np.signbit(blocks[2]))
    assert np.all(np.isfinite(w)) and np.abs(w).max() < 65520 * 8


def test_bf16_bits_round_to_nearest_even():
    """bf16 inputs are the fp32 draws rounded to nearest even: exact values,
    ties to the even pattern, and random values against exact rational
    rounding."""
    from fractions import Fraction as Fr
    cases = {1.0: 0x3F80, -2.0: 0xC000, 1.0 + 2.0 ** -8: 0x3F80, 1.0 + 3 * 2.0 ** -8: 0x3F82,
             1.0 + 2.0 ** -8 + 2.0 ** -20: 0x3F81, 65504.0: 0x4780}
    got = synth.bf16_bits(np.array(list(cases), np.float32))
    assert [int(v) for v in got] == list(cases.values())
    x = np.random.default_rng(0).standard_normal(2000).astype(np.float32)
    b = synth.bf16_bits(x)
    for xv, bv in zip(x, b):
        # neighbouring patterns bracket x; the chosen one is nearest (even on ties)
        lo = int(bv)
        val = (np.array([lo], np.uint32) << 16).view(np.float32)[0]
        err = abs(Fr(float(xv)) - Fr(float(val)))
        for nb in (lo - 1, lo + 1):
            other = (np.array([nb], np.uint32) << 16).view(np.float32)[0]
            e2 = abs(Fr(float(xv)) - Fr(float(other)))
            assert err < e2 or (err == e2 and lo % 2 == 0)
