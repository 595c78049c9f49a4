"""GPU batched-decode GEMV parity against the oracle: every output within
1e-3 * sum|w*x| + 1e-6, exact where the arithmetic is exact, deterministic."""

import numpy as np
import pytest

import oracle
import synth
from _golden import load
from _gpu import assert_matmul_close, to_dev, to_dev_bf16, to_host, workload_weights_cached

pytestmark = pytest.mark.gpu

BLOCKS, _ = load()
TDT = {"f16": np.float16, "f32": np.float32}


def run_gemv(q4, x, packed, n, k, ydt, dev):
    import torch
    ydtype = torch.float16 if ydt == "f16" else torch.float32
    y = q4.q4_gemv(to_dev(x, dev), to_dev(packed, dev), y_dtype=ydtype, n=n, k=k)
    return to_host(y)


def test_golden_worked_dot(q4lib, gpu):
    blk = next(b for b in BLOCKS if b.name == "A")
    packed = oracle.quantize(blk.x[None, :])
    for xdt in ("f16", "f32"):
        y = run_gemv(q4lib, np.ones((1, 32), TDT[xdt]), packed, 1, 32, "f32", gpu)
        assert y[0, 0] == -2.0


@pytest.mark.parametrize("xdt", ["f16", "f32"])
def test_one_hot_rows_give_exact_weights(q4lib, gpu, xdt):
    """x = identity: y[i, n] = (q - 8) * d of element i, exactly (pins the nibble layout)."""
    n, k = 70, 64
    w = synth.random_weights(3, n, k, "student_t")
    packed = oracle.quantize(w)
    deq = oracle.dequantize(packed, n, k)
    for r0 in (0, 32):
        x = np.zeros((32, k), TDT[xdt])
        x[np.arange(32), r0 + np.arange(32)] = 1
        y = run_gemv(q4lib, x, packed, n, k, "f32", gpu)
        assert np.array_equal(y, deq[:, r0:r0 + 32].T)


@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8, 10, 16, 17, 31, 32])
@pytest.mark.parametrize("n,k", [(1, 32), (7, 96), (64, 512), (300, 2080), (129, 5120)])
def test_shapes_f16(q4lib, gpu, m, n, k):
    w = synth.random_weights(m + n + k, n, k, "outlier")
    x = synth.random_activations(m * 3 + k, m, k, "f16")
    packed = oracle.quantize(w)
    g = run_gemv(q4lib, x, packed, n, k, "f16", gpu)
    assert_matmul_close(g, x, packed, n, k, what=f"m{m} n{n} k{k}")


@pytest.mark.parametrize("xdt,ydt", [("f32", "f32"), ("f32", "f16"), ("f16", "f32")])
@pytest.mark.parametrize("m", [1, 4, 13, 32])
def test_dtypes(q4lib, gpu, xdt, ydt, m):
    n, k = 257, 1056
    w = synth.random_weights(5, n, k, "student_t")
    x = synth.random_activations(6 + m, m, k, xdt)
    packed = oracle.quantize(w)
    g = run_gemv(q4lib, x, packed, n, k, ydt, gpu)
    assert_matmul_close(g, x, packed, n, k, what=f"{xdt}->{ydt} m{m}")


def test_edge_case_weights(q4lib, gpu):
    """Every quantiser corner case, including scales far above the fp16 weight range
    (the GEMV keeps q - 8 exact and applies d in fp32)."""
    n, k = 96, 32 * 24
    w = synth.edge_case_weights(7, n, k)
    x = synth.random_activations(8, 10, k, "f16")
    packed = oracle.quantize(w)
    g = run_gemv(q4lib, x, packed, n, k, "f32", gpu)
    assert_matmul_close(g, x, packed, n, k, what="edge")


@pytest.mark.parametrize("wid", [1, 2, 3])
def test_workloads_full(q4lib, gpu, wid):
    """Full-size decode workloads, every output checked, GPU-quantised weights."""
    wl = synth.WORKLOADS[wid]
    lin = wl.linears[0]
    w = workload_weights_cached(wl, lin)
    packed_d = q4lib.q4_quantize(to_dev(w, gpu))
    packed = to_host(packed_d)
    assert np.array_equal(packed[:64], oracle.quantize(w[:64]))
    del w
    for m in wl.ms:
        x = synth.workload_activations(wl, lin.k, m)
        import torch
        y = q4lib.q4_gemv(to_dev(x, gpu), packed_d,
                          y_dtype=torch.float16 if wl.y_dtype == "f16" else torch.float32)
        assert_matmul_close(to_host(y), x, packed, lin.n, lin.k, what=f"{wl.name} m{m}")


def test_layer_workload(q4lib, gpu):
    """All seven linears of the Student-t layer at M = 1 and 10, every output,
    on GPU-quantised weights."""
    import torch
    wl = synth.WORKLOADS[5]
    for lin in wl.linears:
        w = workload_weights_cached(wl, lin)
        packed_d = q4lib.q4_quantize(to_dev(w, gpu))
        packed = to_host(packed_d)
        assert np.array_equal(packed[-16:], oracle.quantize(w[-16:]))
        del w
        for m in (1, 10):
            x = synth.workload_activations(wl, lin.k, m)
            y = to_host(q4lib.q4_gemv(to_dev(x, gpu), packed_d, y_dtype=torch.float16))
            assert_matmul_close(y, x, packed, lin.n, lin.k, what=f"layer/{lin.name} m{m}")


@pytest.mark.parametrize("group", [("q", "k", "v"), ("gate", "up")])
def test_layer_concatenated_projections(q4lib, gpu, group):
    """Linears that read the same activation run as one launch over their packed
    rows stacked (q/k/v: 7168 rows, gate/up: 34816): each weight is quantised
    into its row slice of one buffer, the slices match the oracle's bytes, and
    the one GEMV over the whole buffer is within tolerance of the oracle on
    sampled columns that include both sides of every segment boundary."""
    import torch
    wl = synth.WORKLOADS[5]
    lins = [next(l for l in wl.linears if l.name == nm) for nm in group]
    k = lins[0].k
    assert all(l.k == k for l in lins)
    rows = sum(l.n for l in lins)
    buf = torch.empty((rows, (k // 32) * 18), dtype=torch.uint8, device=gpu)
    r, edges = 0, []
    for lin in lins:
        w = workload_weights_cached(wl, lin)
        q4lib.q4_quantize(to_dev(w, gpu), packed=buf[r:r + lin.n])
        torch.cuda.synchronize()
        assert np.array_equal(to_host(buf[r:r + 8]), oracle.quantize(w[:8]))
        assert np.array_equal(to_host(buf[r + lin.n - 8:r + lin.n]), oracle.quantize(w[-8:]))
        del w
        edges += [r, r + 1, r + lin.n - 2, r + lin.n - 1]
        r += lin.n
    packed = to_host(buf)
    rng = np.random.default_rng(len(group))
    cols = np.unique(np.concatenate([rng.choice(rows, size=1024, replace=False), edges]))
    for m in (1, 10):
        x = synth.workload_activations(wl, k, m)
        y = to_host(q4lib.q4_gemv(to_dev(x, gpu), buf, y_dtype=torch.float16))
        assert y.shape == (m, rows)
        assert_matmul_close(y[:, cols], x, packed, rows, k, cols=cols,
                            what=f"{'+'.join(group)} m{m}")


def test_deterministic(q4lib, gpu):
    import torch
    n, k = 5120, 5120
    packed = q4lib.q4_quantize(to_dev(synth.random_weights(2, n, k, "student_t"), gpu))
    for m in (1, 10, 32):
        x = to_dev(synth.random_activations(m, m, k, "f16"), gpu)
        a = to_host(q4lib.q4_gemv(x, packed, y_dtype=torch.float32))
        b = to_host(q4lib.q4_gemv(x, packed, y_dtype=torch.float32))
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_sliced_activation_rows(q4lib, gpu):
    """A batch given as a row slice of a bigger activation buffer (pointer offset)."""
    import torch
    n, k = 384, 512
    w = synth.random_weights(4, n, k)
    packed = oracle.quantize(w)
    xall = synth.random_activations(9, 40, k, "f16")
    xd = to_dev(xall, gpu)
    y = q4lib.q4_gemv(xd[8:24], to_dev(packed, gpu), y_dtype=torch.float32)
    assert_matmul_close(to_host(y), xall[8:24], packed, n, k, what="slice")


def test_graph_replay_matches_eager(q4lib, gpu):
    """Launches recorded into a HIP graph (as the benchmark times them) give the
    eager result on every replay, with eager work and synchronisation between
    replays."""
    import torch
    n, k = 520, 2048
    w = synth.random_weights(41, n, k, "outlier")
    packed = to_dev(oracle.quantize(w), gpu)
    xs = {m: to_dev(synth.random_activations(40 + m, m, k, "f16"), gpu) for m in (1, 10, 16)}
    eager = {m: to_host(q4lib.q4_gemv(xs[m], packed, n=n, k=k)) for m in xs}
    ys = {m: torch.empty((m, n), dtype=torch.float16, device=gpu) for m in xs}
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for m in xs:
            q4lib.q4_gemv(xs[m], packed, y=ys[m], n=n, k=k)
    for rep in range(4):
        for m in xs:
            ys[m].fill_(float("nan"))
        scratch = q4lib.q4_gemv(xs[16], packed, n=n, k=k)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for m in xs:
            assert np.array_equal(to_host(ys[m]), eager[m]), f"replay {rep} m={m}"
        assert np.array_equal(to_host(scratch), eager[16])


@pytest.mark.parametrize("m", [1, 3, 4, 7, 12, 16])
@pytest.mark.parametrize("n,k", [(4, 512), (5, 512), (1027, 1024), (2051, 3072), (6000, 1536)])
def test_row_group_shapes(q4lib, gpu, m, n, k):
    """Shapes around the four-row grouping: a single group, a ragged last group,
    workgroups whose waves get no task, and task ranges spanning several sets."""
    w = synth.random_weights(7 * m + n + k, n, k, "outlier")
    x = synth.random_activations(5 * m + k, m, k, "f16")
    packed = oracle.quantize(w)
    g = run_gemv(q4lib, x, packed, n, k, "f16", gpu)
    assert_matmul_close(g, x, packed, n, k, what=f"m{m} n{n} k{k}")


@pytest.mark.parametrize("m", [5, 16, 17, 32])
@pytest.mark.parametrize("n,k", [(16, 3072), (4097, 1536), (4097, 3072), (8200, 1536),
                                 (12300, 1536), (16400, 512)])
def test_matrix_core_tile_shapes(q4lib, gpu, m, n, k):
    """The 16x16x32 matrix-core GEMV (m > 4, k a multiple of 512): one to five
    16-row tiles per workgroup, one or two activation tiles, one to six K
    phases, a ragged last row tile."""
    w = synth.random_weights(11 * m + n + k, n, k, "outlier")
    x = synth.random_activations(13 * m + k, m, k, "f16")
    packed = oracle.quantize(w)
    g = run_gemv(q4lib, x, packed, n, k, "f16", gpu)
    assert_matmul_close(g, x, packed, n, k, what=f"m{m} n{n} k{k}")


@pytest.mark.parametrize("m", [5, 16, 17, 32])
@pytest.mark.parametrize("n,k", [(4097, 8192), (1000, 16384)])
def test_matrix_core_tile_rows_spread(q4lib, gpu, m, n, k):
    """K long enough for eight or more phases: rows spread over every compute
    unit, 17 (4097 rows) or 4 (1000 rows) per workgroup, so every workgroup's
    last 16-row tile is partial and its unfilled rows must never be stored."""
    w = synth.random_weights(17 * m + n + k, n, k, "student_t")
    x = synth.random_activations(19 * m + k, m, k, "f16")
    packed = oracle.quantize(w)
    g = run_gemv(q4lib, x, packed, n, k, "f32", gpu)
    assert_matmul_close(g, x, packed, n, k, what=f"m{m} n{n} k{k}")


# bf16 activations: the m <= 4 kernel (k a multiple of 512) converts the
# staged rows in LDS, the tile kernel (m > 4, k a multiple of 512) converts
# each operand fragment, other shapes widen them exactly in the general kernel.
BF16_CASES = [(1, 300, 2048), (2, 129, 5120), (3, 64, 512), (4, 1000, 17408),
              (5, 4097, 1536), (16, 1000, 3072), (17, 520, 2048), (32, 16, 3072),
              (1, 257, 1056), (13, 70, 768), (32, 7, 96), (4, 300, 2080)]


@pytest.mark.parametrize("m,n,k", BF16_CASES)
@pytest.mark.parametrize("ydt", ["f16", "f32"])
def test_bf16_activations(q4lib, gpu, m, n, k, ydt):
    import torch
    w = synth.random_weights(3 * m + n + k, n, k, "student_t")
    xb = synth.random_activations(7 * m + k, m, k, "bf16")
    packed = oracle.quantize(w)
    y = q4lib.q4_gemv(to_dev_bf16(xb, gpu), to_dev(packed, gpu),
                      y_dtype=torch.float16 if ydt == "f16" else torch.float32, n=n, k=k)
    assert_matmul_close(to_host(y), oracle.widen_bf16(xb), packed, n, k,
                        what=f"bf16 m{m} n{n} k{k} -> {ydt}")


@pytest.mark.parametrize("m,k", [(4, 512), (32, 512), (32, 96)])
def test_bf16_one_hot_rows_give_exact_weights(q4lib, gpu, m, k):
    """bf16 x = identity rows: y is the dequantised weight exactly, on each path."""
    n = 70
    w = synth.random_weights(31, n, k, "student_t")
    packed = oracle.quantize(w)
    deq = oracle.dequantize(packed, n, k)
    x = np.zeros((m, k), np.float32)
    x[np.arange(m), np.arange(m)] = 1
    y = to_host(q4lib.q4_gemv(to_dev_bf16(synth.bf16_bits(x), gpu), to_dev(packed, gpu), n=n, k=k))
    assert y.dtype == np.float32  # bf16 activations default to an fp32 output
    assert np.array_equal(y, deq[:, :m].T)


@pytest.mark.parametrize("m", [3, 10])
def test_bf16_activations_across_the_fp16_range(q4lib, gpu, m):
    """bf16 values spanning fp16's normal range (2^-14 .. 60000): the in-kernel
    conversion is exact there, so the result stays within tolerance."""
    n, k = 200, 1024
    rng = np.random.default_rng(m)
    mag = np.exp2(rng.uniform(-14, 15.8, size=(m, k))).astype(np.float32)
    x = np.where(rng.random((m, k)) < 0.5, -mag, mag).astype(np.float32)
    xb = synth.bf16_bits(x)
    w = synth.random_weights(33, n, k, "normal") * np.float32(1e-3)
    packed = oracle.quantize(w)
    y = to_host(q4lib.q4_gemv(to_dev_bf16(xb, gpu), to_dev(packed, gpu), n=n, k=k))
    assert_matmul_close(y, oracle.widen_bf16(xb), packed, n, k, what=f"bf16 range m{m}")


@pytest.mark.parametrize("m,n,k", [(32, 17408, 1024), (17, 20000, 512), (24, 34816, 1024)])
def test_matrix_core_tile_wide_two_activation_tiles(q4lib, gpu, m, n, k):
    """m > 16 with more than 64 rows per compute unit: five row tiles in a slot
    sized for 68 weight rows (the fifth tile's rows past 68 read bytes of the
    activation area and are never stored); 34816 rows take two rounds."""
    w = synth.random_weights(23 * m + n + k, n, k, "student_t")
    x = synth.random_activations(29 * m + k, m, k, "f16")
    packed = oracle.quantize(w)
    g = run_gemv(q4lib, x, packed, n, k, "f32", gpu)
    rng = np.random.default_rng(n)
    cols = np.unique(np.concatenate([rng.choice(n, size=1500, replace=False),
                                     np.arange(0, n, 68), np.arange(67, n, 68), [n - 1]]))
    assert_matmul_close(g[:, cols], x, packed, n, k, cols=cols, what=f"wide m{m} n{n} k{k}")


# Seven- and nine-tile workgroups (m <= 16 and m <= 10): all 16 T rows
# copied (rows past n re-read row n - 1), or fewer (the rest of the slot is
# never stored); one round of workgroups or several; fp16 and bf16 inputs.
SEVEN_NINE_CASES = [(10, 34816, 1024, "f16"), (10, 34816, 5120, "f16"), (7, 28672, 4096, "f16"),
                    (16, 24576, 4096, "f16"), (16, 28000, 1536, "f16"), (9, 40000, 1024, "f16"),
                    (12, 40000, 1024, "f16"), (10, 34816, 1024, "bf16"), (16, 24576, 1536, "bf16")]


@pytest.mark.parametrize("m,n,k,xdt", SEVEN_NINE_CASES)
def test_matrix_core_tile_seven_and_nine_tiles(q4lib, gpu, m, n, k, xdt):
    import torch
    w = synth.random_weights(31 * m + n + k, n, k, "student_t")
    packed = oracle.quantize(w)
    if xdt == "bf16":
        xb = synth.random_activations(37 * m + k, m, k, "bf16")
        y = to_host(q4lib.q4_gemv(to_dev_bf16(xb, gpu), to_dev(packed, gpu), y_dtype=torch.float32,
                                  n=n, k=k))
        x = oracle.widen_bf16(xb)
    else:
        x = synth.random_activations(37 * m + k, m, k, "f16")
        y = run_gemv(q4lib, x, packed, n, k, "f32", gpu)
    rng = np.random.default_rng(n + m)
    cols = np.unique(np.concatenate([rng.choice(n, size=1200, replace=False), np.arange(0, n, 112),
                                     np.arange(111, n, 112), np.arange(135, n, 136),
                                     np.arange(143, n, 144), [n - 1]]))
    assert_matmul_close(y[:, cols], x, packed, n, k, cols=cols, what=f"{xdt} m{m} n{n} k{k}")


# Past one round of nine-tile workgroups (m <= 10, more than 144 rows per
# compute unit): two workgroups per compute unit of 72-112 rows (five to seven
# tiles, the last one partial where the rows are not a multiple of 16), the
# last workgroup ragged; 8-block phases, so k = 512 has two.
PAIR_CASES = [(5, 40000, 1024, "f16"), (10, 45000, 1536, "f16"), (8, 57000, 1024, "f16"),
              (6, 37000, 512, "f16"), (10, 38000, 2048, "bf16"), (9, 40000, 1024, "f16")]


@pytest.mark.parametrize("m,n,k,xdt", PAIR_CASES)
def test_matrix_core_tile_two_workgroups_per_cu(q4lib, gpu, m, n, k, xdt):
    import torch
    w = synth.random_weights(53 * m + n + k, n, k, "student_t")
    packed = oracle.quantize(w)
    if xdt == "bf16":
        xb = synth.random_activations(59 * m + k, m, k, "bf16")
        y = to_host(q4lib.q4_gemv(to_dev_bf16(xb, gpu), to_dev(packed, gpu), y_dtype=torch.float32,
                                  n=n, k=k))
        x = oracle.widen_bf16(xb)
    else:
        x = synth.random_activations(59 * m + k, m, k, "f16")
        y = run_gemv(q4lib, x, packed, n, k, "f32", gpu)
    rows = -(-(-(-n // 512)) // 4) * 4  # ceil(n / 512) rounded up to a multiple of 4
    rng = np.random.default_rng(n + 7 * m)
    cols = np.unique(np.concatenate([rng.choice(n, size=1200, replace=False), np.arange(0, n, rows),
                                     np.arange(rows - 1, n, rows), np.arange(15, n, 16),
                                     np.arange(n - 130, n)]))
    assert_matmul_close(y[:, cols], x, packed, n, k, cols=cols, what=f"{xdt} m{m} n{n} k{k}")


def test_bf16_beyond_fp16_on_two_workgroups_per_cu(q4lib, gpu):
    """The two-workgroups-per-CU form with bf16 activations fp16 cannot hold:
    every workgroup recomputes its rows on the exact route.  Sampled
    outputs, every workgroup's first and last row among them."""
    import torch
    from test_gpu_gemm import bf16_beyond_fp16
    m, n, k = 7, 38100, 1024
    w = synth.random_weights(197, n, k, "student_t")
    packed = oracle.quantize(w)
    xb, _ = bf16_beyond_fp16(199, m, k)
    y = to_host(q4lib.q4_gemv(to_dev_bf16(xb, gpu), to_dev(packed, gpu), y_dtype=torch.float32,
                              n=n, k=k))
    assert np.isfinite(y).all()
    rows = 76
    cols = np.unique(np.concatenate([np.arange(0, n, rows), np.arange(rows - 1, n, rows), [n - 1],
                                     np.random.default_rng(3).choice(n, size=800, replace=False)]))
    assert_matmul_close(y[:, cols], oracle.widen_bf16(xb), packed, n, k, cols=cols,
                        what=f"bf16 range m{m} n{n} k{k}")


@pytest.mark.parametrize("m,n,k", [(4, 5120, 17408), (4, 300, 16384), (3, 1000, 17408), (4, 37, 17920)])
def test_balanced_long_k(q4lib, gpu, m, n, k):
    """m <= 4 with long K: the staged activations (up to 140 KB) leave room for
    a two-task ring per wave only, which the plan then takes."""
    w = synth.random_weights(41 * m + n + k, n, k, "outlier")
    x = synth.random_activations(43 * m + k, m, k, "f16")
    packed = oracle.quantize(w)
    g = run_gemv(q4lib, x, packed, n, k, "f32", gpu)
    cols = np.unique(np.concatenate([np.arange(0, n, 11), [n - 1]]))
    assert_matmul_close(g[:, cols], x, packed, n, k, cols=cols, what=f"m{m} n{n} k{k}")


def test_packed_weight_past_2_gib(q4lib, gpu):
    """A 131072 x 32768 weight: 2.4 GB of packed rows (byte offsets past 2^31),
    quantised on the device from 17 GB of fp32.  Sampled output features, the
    first and last rows among them, match the oracle on their own packed rows
    at m = 1 and 16."""
    import torch
    n, k = 131072, 32768
    g = torch.Generator(device=gpu)
    g.manual_seed(131072)
    w = torch.randn((n, k), device=gpu, generator=g)
    w.mul_(0.02)
    packed_d = q4lib.q4_quantize(w)
    del w
    torch.cuda.empty_cache()
    cols = np.unique(np.concatenate([np.random.default_rng(2).choice(n, 30, replace=False),
                                     [0, 65535, 65536, 119304, n - 1]]))
    packed_cols = to_host(packed_d.index_select(0, torch.from_numpy(cols).to(gpu)))
    for m in (1, 16):
        x = synth.random_activations(m + 131, m, k, "f16")
        y = to_host(q4lib.q4_gemv(to_dev(x, gpu), packed_d, y_dtype=torch.float32))
        assert np.isfinite(y).all()
        assert_matmul_close(y[:, cols], x, packed_cols, len(cols), k, what=f"{n}x{k} m{m}")


def cancellation_case(m, k, n=64):
    """Blocks whose one nonzero weight meets a tiny activation while every zero
    weight meets a large one.  Row r has weight +-1.0 at element r % 4 of each
    block (code 0, with d = -0.125 or +0.125) and 0 elsewhere (code 8);
    activations are 2^-10 (j + 1) at elements j < 4 and +-1024 at the
    other 28, so y is a sum of the tiny terms only: a kernel whose error
    scales with sum |x| rather than sum |x w| loses them entirely."""
    w = np.zeros((n, k), np.float32)
    for r in range(n):
        w[r, (r % 4)::32] = 1.0 if (r // 4) % 2 == 0 else -1.0
    x = np.empty((m, k), np.float32)
    for i in range(m):
        big = np.float32(1024.0 if i % 2 == 0 else -1024.0)
        x[i] = big
        for j in range(4):
            sgn = np.where((np.arange(k // 32) + i + j) % 3 == 0, -1.0, 1.0).astype(np.float32)
            x[i, j::32] = np.float32(2.0 ** -10 * (j + 1)) * sgn
    return w, x


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
@pytest.mark.parametrize("k", [512, 768, 5120])
@pytest.mark.parametrize("m", [1, 4, 5, 10, 16, 32])
def test_large_activations_on_zero_weights(q4lib, gpu, m, k, xdt):
    """Every kernel (balanced m <= 4, matrix-core tile 5 <= m <= 32 at k % 512
    == 0, streaming at k = 768) keeps the tiny products of the cancellation
    case: every output within 1e-3 * sum|w*x| + 1e-6 of the oracle."""
    import torch
    n = 64
    w, x32 = cancellation_case(m, k, n)
    packed = oracle.quantize(w)
    if xdt == "f16":
        x = x32.astype(np.float16)
        xd, xref = to_dev(x, gpu), x
    else:
        xb = synth.bf16_bits(x32)
        xd, xref = to_dev_bf16(xb, gpu), oracle.widen_bf16(xb)
    for ydt in (torch.float32, torch.float16):
        y = to_host(q4lib.q4_gemv(xd, to_dev(packed, gpu), y_dtype=ydt, n=n, k=k))
        y_ref, _ = oracle.matmul_ref(xref, packed, n, k)
        assert np.abs(y_ref).min() > 0  # the tiny terms are the whole result
        assert_matmul_close(y, xref, packed, n, k, what=f"cancel m{m} k{k} {xdt} {ydt}")


def wide_range_f16(seed, m, k):
    """fp16 activations whose magnitudes span the whole fp16 range, subnormals
    2^-24 .. 2^-15 and exact zeros included, with random signs."""
    rng = np.random.default_rng(seed)
    e = rng.uniform(-24.0, 15.99, size=(m, k))
    x = np.exp2(e).astype(np.float32)
    x = np.where(rng.random((m, k)) < 0.5, -x, x).astype(np.float16)
    x[rng.random((m, k)) < 0.02] = 0
    return x


@pytest.mark.parametrize("m", [1, 4, 5, 10, 16, 32])
@pytest.mark.parametrize("k", [1536, 5120])
def test_edge_case_weights_main_kernels(q4lib, gpu, m, k):
    """The quantiser's corner-case blocks (zero, -0, ties, constants, subnormal
    and zero scales, scales near the top of the domain, spikes, exact
    multiples, maxima at the last index) through the balanced (m <= 4) and
    matrix-core tile (m >= 5) kernels, with N(0, 1) and with wide-range fp16
    activations; every output checked."""
    n = 300
    w = synth.edge_case_weights(101 + k, n, k)
    packed = oracle.quantize(w)
    for name, x in (("normal", synth.random_activations(103 + m, m, k, "f16")),
                    ("wide", wide_range_f16(107 + m + k, m, k))):
        g = run_gemv(q4lib, x, packed, n, k, "f32", gpu)
        assert_matmul_close(g, x, packed, n, k, what=f"edge {name} m{m} k{k}")


@pytest.mark.parametrize("m", [1, 4, 5, 16, 32])
def test_wide_range_activations(q4lib, gpu, m):
    """Wide-range fp16 activations on ordinary Student-t weights, every kernel
    family: balanced / tile (k = 5120), streaming (k = 768), general (k = 96)."""
    for n, k in ((520, 5120), (130, 768), (33, 96)):
        w = synth.random_weights(109 + m + k, n, k, "student_t")
        x = wide_range_f16(113 + m + k, m, k)
        packed = oracle.quantize(w)
        g = run_gemv(q4lib, x, packed, n, k, "f32", gpu)
        assert_matmul_close(g, x, packed, n, k, what=f"wide m{m} n{n} k{k}")


@pytest.mark.parametrize("m,n,k", [(1, 300, 2048), (3, 1000, 5120), (4, 129, 512),
                                   (5, 4097, 1536), (10, 5120, 5120), (16, 300, 1024),
                                   (32, 520, 2048), (7, 70, 96)])
def test_bf16_activations_beyond_the_fp16_range(q4lib, gpu, m, n, k):
    """bf16 activations fp16 cannot hold (up to 1e20, down to 1e-30, between
    fp16 subnormals): the balanced (m <= 4) and tile (m >= 5) kernels detect
    the inexact conversion and recompute the workgroup's rows on the exact
    route; the general kernel (k = 96) widens exactly anyway.  Every output."""
    import torch
    from test_gpu_gemm import bf16_beyond_fp16
    w = synth.random_weights(181 + k, n, k, "student_t")
    packed = oracle.quantize(w)
    xb, _ = bf16_beyond_fp16(191 + m, m, k)
    y = to_host(q4lib.q4_gemv(to_dev_bf16(xb, gpu), to_dev(packed, gpu), y_dtype=torch.float32,
                              n=n, k=k))
    assert np.isfinite(y).all()
    assert_matmul_close(y, oracle.widen_bf16(xb), packed, n, k, what=f"bf16 range m{m} n{n} k{k}")
