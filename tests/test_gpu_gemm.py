"""GPU prefill GEMM parity against the oracle: every checked output within
1e-3 * sum|w*x| + 1e-6; chunked prefill and whole-batch both in tolerance;
deterministic."""

import numpy as np
import pytest

import oracle
import synth
from _gpu import (assert_matmul_close, sample_rows, to_dev, to_dev_bf16, to_host,
                  workload_weights_cached)

pytestmark = pytest.mark.gpu


def ytorch(ydt):
    import torch
    return torch.float16 if ydt == "f16" else torch.float32


def run_gemm(q4, x, packed, n, k, ydt, dev):
    y = q4.q4_gemm(to_dev(x, dev), to_dev(packed, dev), y_dtype=ytorch(ydt), n=n, k=k)
    return to_host(y)


@pytest.mark.parametrize("m", [1, 33, 128, 200, 257, 640])
@pytest.mark.parametrize("n,k", [(1, 32), (100, 64), (128, 96), (300, 544), (129, 5120), (520, 2080)])
def test_shapes(q4lib, gpu, m, n, k):
    w = synth.random_weights(m + n + k, n, k, "student_t")
    x = synth.random_activations(m * 5 + k, m, k, "f16")
    packed = oracle.quantize(w)
    g = run_gemm(q4lib, x, packed, n, k, "f16", gpu)
    assert_matmul_close(g, x, packed, n, k, what=f"m{m} n{n} k{k}")


@pytest.mark.parametrize("m", [64, 300])
def test_fp32_output(q4lib, gpu, m):
    n, k = 200, 1024
    w = synth.random_weights(8, n, k, "outlier")
    x = synth.random_activations(9, m, k, "f16")
    packed = oracle.quantize(w)
    g = run_gemm(q4lib, x, packed, n, k, "f32", gpu)
    assert_matmul_close(g, x, packed, n, k, what=f"f32 out m{m}")


def test_one_hot_rows_select_weights(q4lib, gpu):
    """x = identity: y[i, n] is element i's weight (fp16-rounded), pinning the nibble layout."""
    n, k = 96, 128
    w = synth.random_weights(5, n, k, "student_t")
    packed = oracle.quantize(w)
    x = np.eye(k, dtype=np.float16)
    g = run_gemm(q4lib, x, packed, n, k, "f32", gpu)
    assert_matmul_close(g, x, packed, n, k, what="one-hot")


def test_edge_case_weights(q4lib, gpu):
    """Every quantiser corner case whose dequantised weights fit fp16 (|w| <= 65504)."""
    n, k = 96, 32 * 24
    w = synth.edge_case_weights(7, n, k, top=65504.0)
    x = synth.random_activations(8, 160, k, "f16")
    packed = oracle.quantize(w)
    g = run_gemm(q4lib, x, packed, n, k, "f32", gpu)
    assert_matmul_close(g, x, packed, n, k, what="edge")


def test_prefill_chunked_and_whole(q4lib, gpu):
    """2048 prompt rows as one batch and as 8 chunks of 256 (pointer offsets):
    every one of the 2048 x 17408 outputs of both runs against the oracle."""
    import torch
    wl = synth.WORKLOADS[4]
    lin = wl.linears[0]
    w = workload_weights_cached(wl, lin)
    packed_d = q4lib.q4_quantize(to_dev(w, gpu))
    packed = to_host(packed_d)
    assert np.array_equal(packed[:16], oracle.quantize(w[:16]))
    del w
    x = synth.workload_activations(wl, lin.k, 2048)
    xd = to_dev(x, gpu)
    whole = q4lib.q4_gemm(xd, packed_d, y_dtype=torch.float16)
    chunked = torch.empty_like(whole)
    for c in range(8):
        q4lib.q4_gemm(xd[c * 256:(c + 1) * 256], packed_d, y=chunked[c * 256:(c + 1) * 256])
    y_ref, S = oracle.matmul_ref(x, packed, lin.n, lin.k)
    for name, y in (("whole", whole), ("chunked", chunked)):
        ok, worst, idx = oracle.check(to_host(y), y_ref, S)
        assert ok, f"{wl.name}/{name}: worst |gpu-oracle|/bound = {worst:.3g} at {idx}"
    again = q4lib.q4_gemm(xd, packed_d, y_dtype=torch.float16)
    assert torch.equal(again.view(torch.int16), whole.view(torch.int16))


def test_layer_workload(q4lib, gpu):
    """All seven Student-t linears of the layer: at M = 256 every output; at
    M = 4096 a seeded set of at least 512 full rows per linear (over 12.5 % of
    the rows, both sides of every 256-row tile boundary among them) against the oracle."""
    import torch
    wl = synth.WORKLOADS[5]
    for lin in wl.linears:
        w = workload_weights_cached(wl, lin)
        packed_d = q4lib.q4_quantize(to_dev(w, gpu))
        packed = to_host(packed_d)
        del w
        for m in (256, 4096):
            x = synth.workload_activations(wl, lin.k, m)
            y = to_host(q4lib.q4_gemm(to_dev(x, gpu), packed_d, y_dtype=torch.float16))
            if m == 256:
                rows = np.arange(m)
            else:
                rows = np.unique(np.concatenate([sample_rows(m, 512, m + lin.tensor_id),
                                                 np.arange(255, m, 256), np.arange(0, m, 256)]))
                assert len(rows) >= 512
            assert_matmul_close(y[rows], x[rows], packed, lin.n, lin.k,
                                what=f"layer/{lin.name} m{m}")


def test_long_ragged_prefill_sampled(q4lib, gpu):
    """8191 prompt rows (the last 256-row tile one row short) on the 5120 x 5120
    projection, fp16 output: sampled rows, the first and last of every
    row-tile boundary among them, against the oracle."""
    import torch
    wl = synth.WORKLOADS[2]
    lin = wl.linears[0]
    w = workload_weights_cached(wl, lin)
    packed_d = q4lib.q4_quantize(to_dev(w, gpu))
    packed = to_host(packed_d)
    del w
    m = 8191
    x = synth.random_activations(81, m, lin.k, "f16")
    y = to_host(q4lib.q4_gemm(to_dev(x, gpu), packed_d, y_dtype=torch.float16))
    assert np.isfinite(y).all()
    rows = np.unique(np.concatenate([sample_rows(m, 8, 7), [0, 255, 256, 4095, 4096, 7935, 7936, m - 1]]))
    assert_matmul_close(y[rows], x[rows], packed, lin.n, lin.k, what=f"{wl.name} m{m}")


@pytest.mark.parametrize("m", [300, 1100])
def test_long_k_sampled(q4lib, gpu, m):
    """k = 65536 (2048 Q4_0 blocks per row) on the slice-K tile (m = 300) and
    the 256 x 256 tile (m = 1100), ragged n: sampled rows against the oracle."""
    import torch
    n, k = 700, 65536
    w = synth.random_weights(65, n, k, "normal")
    packed_d = q4lib.q4_quantize(to_dev(w, gpu))
    packed = to_host(packed_d)
    del w
    x = synth.random_activations(m + 65, m, k, "f16")
    y = to_host(q4lib.q4_gemm(to_dev(x, gpu), packed_d, y_dtype=torch.float32))
    assert np.isfinite(y).all()
    rows = sample_rows(m, 8, m)
    assert_matmul_close(y[rows], x[rows], packed, n, k, what=f"{m}x{n}x{k}")


def test_deterministic(q4lib, gpu):
    import torch
    n, k = 3000, 5120
    packed = q4lib.q4_quantize(to_dev(synth.random_weights(2, n, k), gpu))
    x = to_dev(synth.random_activations(3, 700, k, "f16"), gpu)
    a = q4lib.q4_gemm(x, packed, y_dtype=torch.float32)
    b = q4lib.q4_gemm(x, packed, y_dtype=torch.float32)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_largest_fp16_scale(q4lib, gpu):
    """Blocks whose scale is the largest the fp16 dequant path accepts (|d| = 8188)."""
    n, k = 40, 256
    w = synth.random_weights(21, n, k) * np.float32(1e5)
    w = np.clip(w, -65504, 65504).astype(np.float32)
    w[:, ::32] = np.float32(65504) * np.sign(w[:, ::32] + np.float32(0.5))
    packed = oracle.quantize(w)
    d, _ = oracle.unpack(packed, n, k)
    assert np.abs(d.astype(np.float32)).max() == 8188
    x = synth.random_activations(22, 70, k, "f16") * np.float16(0.01)
    g = run_gemm(q4lib, x, packed, n, k, "f32", gpu)
    assert np.all(np.isfinite(g))
    assert_matmul_close(g, x, packed, n, k, what="largest scale")


def test_graph_replay_matches_eager(q4lib, gpu):
    """A graph of GEMM launches (as the benchmark times them) reproduces the
    eager result on every replay."""
    import torch
    m, n, k = 300, 384, 1024
    w = synth.random_weights(43, n, k, "normal")
    packed = to_dev(oracle.quantize(w), gpu)
    x = to_dev(synth.random_activations(44, m, k, "f16"), gpu)
    eager = to_host(q4lib.q4_gemm(x, packed, n=n, k=k))
    work = torch.empty(max(q4lib.q4_gemm_workspace_size(m, n, k), 1), dtype=torch.uint8,
                       device=gpu)
    y = torch.empty((m, n), dtype=torch.float16, device=gpu)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q4lib.q4_gemm(x, packed, y=y, workspace=work, n=n, k=k)
    for rep in range(3):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(y), eager), f"replay {rep}"


@pytest.mark.parametrize("m,n,k", [(300, 11000, 256), (1100, 14000, 128), (256, 17408, 512),
                                   (2048, 17408, 64), (1030, 13200, 1024)])
def test_main_and_tail_launches(q4lib, gpu, m, n, k):
    """Shapes whose tile count leaves a partial round on 256 compute units: the
    leading columns go to the main tiles in whole rounds, the rest to tiles
    with K split across workgroups (fp32 partials in the workspace, then a
    fixed-order reduction); 1030 x 13200 x 1024 puts slice-K tail tiles
    behind 256 x 256 main tiles.  Every output is checked."""
    w = synth.random_weights(3 * m + n + k, n, k, "student_t")
    x = synth.random_activations(7 * m + k, m, k, "f16")
    packed = oracle.quantize(w)
    g = run_gemm(q4lib, x, packed, n, k, "f16", gpu)
    assert_matmul_close(g, x, packed, n, k, what=f"m{m} n{n} k{k}")


@pytest.mark.parametrize("m,n,k", [(1, 100, 1024), (33, 4097, 1280), (129, 300, 2048), (255, 1000, 1536),
                                   (300, 11000, 1024), (700, 9000, 3072)])
def test_slice_k_tiles(q4lib, gpu, m, n, k):
    """m < 1024, k % 256 == 0, k >= 1024: 128 x 128 tiles whose four waves each
    take one k16 slice of every step; ragged rows and columns, an odd number of
    256-wide weight segments (k = 1280), a split-K tail whose splits hold one
    segment each (300 x 11000 x 1024) and a launch with no tail (700 x 9000)."""
    w = synth.random_weights(5 * m + n + k, n, k, "student_t")
    x = synth.random_activations(11 * m + k, m, k, "f16")
    packed = oracle.quantize(w)
    g = run_gemm(q4lib, x, packed, n, k, "f32", gpu)
    assert_matmul_close(g, x, packed, n, k, what=f"m{m} n{n} k{k}")


@pytest.mark.parametrize("m,n,k", [(37, 70, 96), (64, 300, 1024), (256, 1000, 2048),
                                   (300, 11000, 1024), (1030, 2100, 1024)])
def test_bf16_activations(q4lib, gpu, m, n, k):
    """bf16 activations staged as fp16 in the workspace, then every GEMM path:
    the output-split kernel (k % 64 != 0), slice-K tiles, 256 x 256 tiles with
    a split-K tail; sampled rows for the larger shapes."""
    import torch
    w = synth.random_weights(5 * m + n + k, n, k, "student_t")
    xb = synth.random_activations(3 * m + k, m, k, "bf16")
    packed = oracle.quantize(w)
    need16 = q4lib.q4_gemm_workspace_size(m, n, k)
    needb = q4lib.q4_gemm_workspace_size_dt(m, n, k, q4lib.Q4_BF16)
    assert needb >= need16 + m * k * 2
    y = to_host(q4lib.q4_gemm(to_dev_bf16(xb, gpu), to_dev(packed, gpu), y_dtype=torch.float32,
                              n=n, k=k))
    rows = sample_rows(m, 96, m + n)
    x = oracle.widen_bf16(xb)
    assert_matmul_close(y[rows], x[rows], packed, n, k, what=f"bf16 m{m} n{n} k{k}")


def test_bf16_chunked_matches_oracle(q4lib, gpu):
    """Row chunks of a bf16 prompt by pointer offset, one shared workspace."""
    import torch
    m, n, k, cs = 512, 2048, 2048, 128
    w = synth.random_weights(77, n, k, "normal")
    xb = synth.random_activations(78, m, k, "bf16")
    packed_d = to_dev(oracle.quantize(w), gpu)
    xd = to_dev_bf16(xb, gpu)
    y = torch.empty((m, n), dtype=torch.float16, device=gpu)
    ws = torch.empty(q4lib.q4_gemm_workspace_size_dt(cs, n, k, q4lib.Q4_BF16), dtype=torch.uint8,
                     device=gpu)
    for c in range(m // cs):
        q4lib.q4_gemm(xd[c * cs:(c + 1) * cs], packed_d, y=y[c * cs:(c + 1) * cs], workspace=ws)
    rows = sample_rows(m, 64, 5)
    assert_matmul_close(to_host(y)[rows], oracle.widen_bf16(xb)[rows], to_host(packed_d), n, k,
                        what="bf16 chunks")


def wide_range_f16(seed, m, k):
    """fp16 activations whose magnitudes span the whole fp16 range, subnormals
    2^-24 .. 2^-15 and exact zeros included, with random signs."""
    rng = np.random.default_rng(seed)
    e = rng.uniform(-24.0, 15.99, size=(m, k))
    x = np.exp2(e).astype(np.float32)
    x = np.where(rng.random((m, k)) < 0.5, -x, x).astype(np.float16)
    x[rng.random((m, k)) < 0.02] = 0
    return x


def edge_rows(seed, n, k, top):
    """n rows of quantiser corner-case blocks: 96 generated rows repeated (the
    block patterns cycle along each row, so repeats stay varied)."""
    base = synth.edge_case_weights(seed, 96, k, top=top)
    reps = (n + 95) // 96
    return np.ascontiguousarray(np.tile(base, (reps, 1))[:n])


# (m, n, k): slice-K tiles (m < 1024, k % 256 == 0, k >= 1024), with and
# without a split-K tail; 256 x 256 tiles with a split-K tail (m >= 1024).
EDGE_GEMM = [(256, 4100, 1536), (700, 6000, 5120), (1100, 4100, 1536), (2048, 8448, 5120)]


@pytest.mark.parametrize("m,n,k", EDGE_GEMM)
def test_edge_case_weights_main_kernels(q4lib, gpu, m, n, k):
    """The quantiser's corner-case blocks (those whose dequantised weights fit
    fp16) through the slice-K, 256 x 256 and split-K tail kernels, with N(0, 1)
    and with wide-range fp16 activations; every output checked."""
    w = edge_rows(131 + k, n, k, 65504.0)
    packed = oracle.quantize(w)
    del w
    pd = to_dev(packed, gpu)
    for name, x in (("normal", synth.random_activations(137 + m, m, k, "f16")),
                    ("wide", wide_range_f16(139 + m + k, m, k))):
        import torch
        g = to_host(q4lib.q4_gemm(to_dev(x, gpu), pd, y_dtype=torch.float32, n=n, k=k))
        assert_matmul_close(g, x, packed, n, k, what=f"edge {name} m{m} n{n} k{k}")


@pytest.mark.parametrize("m,n,k", [(1, 100, 64), (37, 300, 1056), (300, 520, 2048),
                                   (1100, 700, 1024), (256, 200, 96)])
@pytest.mark.parametrize("ydt", ["f16", "f32"])
def test_fp32_activations(q4lib, gpu, m, n, k, ydt):
    """fp32 activations take the exact route (activations and dequantised
    weights in fp32 on fp32 matrix cores); every output checked."""
    w = synth.random_weights(17 * m + n + k, n, k, "student_t")
    x = synth.random_activations(19 * m + k, m, k, "f32")
    packed = oracle.quantize(w)
    g = run_gemm(q4lib, x, packed, n, k, ydt, gpu)
    assert_matmul_close(g, x, packed, n, k, what=f"fp32 x m{m} n{n} k{k} -> {ydt}")


# Every GEMM kernel: the generic kernel (k % 64 != 0), 128 x 128 output-split
# tiles (k = 768), slice-K tiles with and without a split-K tail, 256 x 256
# tiles with a split-K tail.
ALL_GEMM_KERNELS = [(160, 300, 96 * 3), (200, 300, 768), (256, 4100, 1536), (300, 11000, 1024),
                    (1100, 4100, 1536), (2048, 8448, 5120)]


@pytest.mark.parametrize("m,n,k", ALL_GEMM_KERNELS)
def test_scales_beyond_the_fp16_weight_range(q4lib, gpu, m, n, k):
    """Block scales far above 8188 (weights up to 5e5, the top of the domain):
    the fp16 dequantised tile overflows there, the tile's accumulators come out
    non-finite and the workgroup recomputes its tile on the exact route.
    Corner-case rows (a tenth of the blocks near the top of the domain) and a
    weight whose every block is beyond fp16; every output checked."""
    import torch
    for name, w in (("edge", edge_rows(151 + k, n, k, 5.0e5)),
                    ("all-big", np.clip(synth.random_weights(157 + k, n, k, "normal") * np.float32(5e6),
                                        -5e5, 5e5).astype(np.float32))):
        packed = oracle.quantize(w)
        d, _ = oracle.unpack(packed, n, k)
        assert np.abs(d.astype(np.float32)).max() > 8188
        x = synth.random_activations(163 + m, m, k, "f16")
        g = to_host(q4lib.q4_gemm(to_dev(x, gpu), to_dev(packed, gpu), y_dtype=torch.float32,
                                  n=n, k=k))
        assert np.isfinite(g).all()
        assert_matmul_close(g, x, packed, n, k, what=f"big d {name} m{m} n{n} k{k}")


def bf16_beyond_fp16(seed, m, k):
    """bf16 activations, N(0, 1) except in a few rows that also hold values
    fp16 cannot represent: magnitudes up to 1e20 and down to 1e-30, and values
    between fp16 subnormals."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k)).astype(np.float32)
    rows = np.unique(np.concatenate([[0, m - 1], rng.choice(m, size=min(m, 5), replace=False)]))
    for i, r in enumerate(rows):
        cols = rng.choice(k, size=min(k, 9), replace=False)
        kind = i % 3
        if kind == 0:
            x[r, cols] = np.float32(1e20) * rng.uniform(0.5, 1.0, size=len(cols)).astype(np.float32)
        elif kind == 1:
            x[r, cols] = np.float32(1e-30) * rng.uniform(0.5, 1.0, size=len(cols)).astype(np.float32)
        else:
            x[r, cols] = np.float32(1.5 * 2.0 ** -25)   # halfway between fp16 subnormals
        x[r, cols] *= np.where(rng.random(len(cols)) < 0.5, -1, 1).astype(np.float32)
    return synth.bf16_bits(x), rows


@pytest.mark.parametrize("m,n,k", ALL_GEMM_KERNELS)
def test_bf16_activations_beyond_the_fp16_range(q4lib, gpu, m, n, k):
    """bf16 rows holding values fp16 cannot represent are staged as NaN rows, so
    every tile and K split that reads them is recomputed on the exact route
    from the bf16 values; every output checked (rows with 1e20 give outputs
    near 1e19, so the output is fp32)."""
    import torch
    w = synth.random_weights(167 + k, n, k, "student_t")
    packed = oracle.quantize(w)
    xb, rows = bf16_beyond_fp16(173 + m, m, k)
    y = to_host(q4lib.q4_gemm(to_dev_bf16(xb, gpu), to_dev(packed, gpu), y_dtype=torch.float32,
                              n=n, k=k))
    assert np.isfinite(y).all()
    assert_matmul_close(y, oracle.widen_bf16(xb), packed, n, k, what=f"bf16 range m{m} n{n} k{k}")


# Launches with fewer tiles than compute units, split along K on every tile:
# slice-K tiles (the 256-row chunk's k/v and down projections, a 64-row and a
# one-row prompt), 256 x 256 tiles (m >= 1024, k % 256 != 0), output-split
# 128 x 128 tiles (k % 256 != 0, down to one 64-wide k step per split);
# slice-K main tiles plus a split tail at m >= 1024 where 256 x 256 tiles
# would under-fill the chip; one round of slice-K tiles at m = 4096.
SPLIT_EVERY_TILE = [(256, 1024, 5120), (256, 5120, 17408), (64, 768, 2048), (1, 1024, 5120),
                    (1100, 1024, 1088), (2048, 520, 4160), (200, 512, 4160), (100, 300, 1600),
                    (1500, 3000, 1024), (4096, 1024, 5120)]


@pytest.mark.parametrize("m,n,k", SPLIT_EVERY_TILE)
def test_split_every_tile(q4lib, gpu, m, n, k):
    """Every output against the oracle (fp16 and fp32 output), the workspace
    the plan needs, and bit-identical results on a second run."""
    import torch
    w = synth.random_weights(197 * m + n + k, n, k, "student_t")
    x = synth.random_activations(199 * m + k, m, k, "f16")
    packed = oracle.quantize(w)
    xd, pd = to_dev(x, gpu), to_dev(packed, gpu)
    need = q4lib.q4_gemm_workspace_size(m, n, k)
    if (m, n, k) != (4096, 1024, 5120):
        assert need > 0, "expected a split plan"
    for ydt in (torch.float32, torch.float16):
        a = q4lib.q4_gemm(xd, pd, y_dtype=ydt, n=n, k=k)
        b = q4lib.q4_gemm(xd, pd, y_dtype=ydt, n=n, k=k)
        assert torch.equal(a.view(torch.int16 if ydt == torch.float16 else torch.int32),
                           b.view(torch.int16 if ydt == torch.float16 else torch.int32))
        assert_matmul_close(to_host(a), x, packed, n, k, what=f"split m{m} n{n} k{k} {ydt}")
