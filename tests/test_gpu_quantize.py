"""GPU quantiser parity: packed bytes bit-identical to the oracle's."""

import numpy as np
import pytest

import oracle
import synth
from _golden import load
from _gpu import to_dev, to_host, workload_weights_cached

pytestmark = pytest.mark.gpu

BLOCKS, _ = load()


def gpu_quantize(q4, w, dev):
    return to_host(q4.q4_quantize(to_dev(w, dev)))


def test_golden_blocks(q4lib, gpu):
    w = np.stack([b.x for b in BLOCKS])
    packed = gpu_quantize(q4lib, w, gpu)
    for i, b in enumerate(BLOCKS):
        assert packed[i].tobytes().hex() == b.hex, b.name


def test_golden_blocks_fp16(q4lib, gpu):
    rows = [b for b in BLOCKS if np.array_equal(b.x.astype(np.float16).astype(np.float32), b.x)]
    w = np.stack([b.x for b in rows]).astype(np.float16)
    packed = gpu_quantize(q4lib, w, gpu)
    for i, b in enumerate(rows):
        assert packed[i].tobytes().hex() == b.hex, b.name


@pytest.mark.parametrize("n,k", [(1, 32), (3, 96), (17, 512), (64, 5120), (5, 17408), (33, 2080)])
@pytest.mark.parametrize("dist", ["normal", "outlier", "student_t"])
@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_shapes(q4lib, gpu, n, k, dist, dt):
    w = synth.random_weights(n + k, n, k, dist)
    if dt == "f16":
        w = w.astype(np.float16)
    assert np.array_equal(gpu_quantize(q4lib, w, gpu), oracle.quantize(w))


@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_edge_case_blocks(q4lib, gpu, dt):
    w = synth.edge_case_weights(4, 96, 32 * 40, top=65504.0 if dt == "f16" else 5.0e5)
    if dt == "f16":
        w = w.astype(np.float16)
    got = gpu_quantize(q4lib, w, gpu)
    want = oracle.quantize(w)
    bad = np.nonzero(np.any(got.reshape(-1, 18) != want.reshape(-1, 18), axis=1))[0]
    assert bad.size == 0, f"{bad.size} blocks differ, first {bad[:5]}"


@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_workload_weights_bit_exact(q4lib, gpu, wid):
    """Every packed byte of every workload's weights, at full size."""
    wl = synth.WORKLOADS[wid]
    for lin in wl.linears:
        w = workload_weights_cached(wl, lin)
        got = gpu_quantize(q4lib, w, gpu)
        step = 2048
        for r0 in range(0, lin.n, step):
            want = oracle.quantize(w[r0:r0 + step])
            assert np.array_equal(got[r0:r0 + step], want), f"{wl.name}/{lin.name} rows {r0}+"


def test_deterministic(q4lib, gpu):
    w = to_dev(synth.random_weights(1, 256, 5120, "student_t"), gpu)
    a = to_host(q4lib.q4_quantize(w))
    b = to_host(q4lib.q4_quantize(w))
    assert np.array_equal(a, b)


@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_codes_at_rounding_boundaries(q4lib, gpu, dt):
    """Elements within a few ulps of the points where x / d + 8.5 crosses an
    integer (x / d = j + 1/2), for scales across the fp16 range: the code then
    depends on the correctly rounded quotient and on the rounded addition, so
    any quotient that is merely close would change some of these bytes."""
    rng = np.random.default_rng(11)
    nblk = 4096
    # scales: random fp16 values, normal and subnormal
    e = rng.integers(-24, 12, nblk)
    d = (rng.integers(1024, 2048, nblk).astype(np.float64) * 2.0 ** (e - 10)).astype(np.float16)
    d = np.where(d == 0, np.float16(2.0 ** -24), d).astype(np.float32)
    j = rng.integers(-8, 8, (nblk, 32)).astype(np.float64) + 0.5
    ulps = rng.integers(-3, 4, (nblk, 32)).astype(np.float64)
    x = (j * d[:, None] * (1.0 + ulps * 2.0 ** -24)).astype(np.float32)
    x[:, 0] = -8.0 * d  # pins the scale: m / -8 = d exactly
    if dt == "f16":
        x = x.astype(np.float16)
        x[:, 0] = (-8.0 * d).astype(np.float16)
    w = x.reshape(64, 64 * 32)
    got = gpu_quantize(q4lib, w, gpu)
    want = oracle.quantize(w)
    bad = np.nonzero(np.any(got.reshape(-1, 18) != want.reshape(-1, 18), axis=1))[0]
    assert bad.size == 0, f"{bad.size} blocks differ, first {bad[:5]}"


@pytest.mark.parametrize("n,k", [(3, 96), (17, 512), (64, 5120), (33, 2080)])
@pytest.mark.parametrize("dist", ["normal", "student_t"])
def test_bf16_weights(q4lib, gpu, n, k, dist):
    """bf16 weights are widened exactly to fp32 and quantised by the same rule."""
    from _gpu import to_dev_bf16
    wb = synth.bf16_bits(synth.random_weights(n + 2 * k, n, k, dist))
    got = to_host(q4lib.q4_quantize(to_dev_bf16(wb, gpu)))
    assert np.array_equal(got, oracle.quantize(oracle.widen_bf16(wb)))


def test_bf16_edge_case_weights(q4lib, gpu):
    from _gpu import to_dev_bf16
    n, k = 96, 32 * 24
    wb = synth.bf16_bits(synth.edge_case_weights(7, n, k))
    got = to_host(q4lib.q4_quantize(to_dev_bf16(wb, gpu)))
    assert np.array_equal(got, oracle.quantize(oracle.widen_bf16(wb)))


def test_more_than_2_31_elements(q4lib, gpu):
    """A 65537 x 32768 fp32 weight (2^31 + 32768 elements, 8.6 GB): element and
    byte offsets pass 2^31 and 2^32.  Rows on both sides of element 2^31 (row
    65536 starts there) and spread over the weight match the oracle byte for
    byte.  The weight is drawn on the device; only sampled rows come back."""
    import torch
    n, k = 65537, 32768
    g = torch.Generator(device=gpu)
    g.manual_seed(2 ** 31 + 1)
    w = torch.randn((n, k), device=gpu, generator=g)
    w[-1, :64] = torch.tensor([0.0] * 32 + [-1e-30] * 31 + [3.0], device=gpu)  # odd blocks at the end
    packed = q4lib.q4_quantize(w)
    rows = np.unique(np.concatenate([np.random.default_rng(231).choice(n, 12, replace=False),
                                     [0, 32767, 32768, 65534, 65535, 65536]]))
    rows_t = torch.from_numpy(rows).to(gpu)
    w_rows = w.index_select(0, rows_t).cpu().numpy()
    p_rows = packed.index_select(0, rows_t).cpu().numpy()
    del w, packed
    torch.cuda.empty_cache()
    want = oracle.quantize(w_rows)
    assert np.array_equal(p_rows, want), [int(r) for r, a, b in zip(rows, p_rows, want)
                                          if not np.array_equal(a, b)]
