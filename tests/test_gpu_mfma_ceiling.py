"""The benchmark's matrix-core ceiling kernel (libq4floor, q4_mfma_ceiling)
does the products its header states: the sum of every thread's output equals
the sum of all the matrix products' outputs, computed here in float64 from the
header's definition of the LDS values and fragment reads, and every wave of
every workgroup produces the same per-lane values."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def lds_values(seed):
    """The 32768 fp16 values the header defines, as float64."""
    i = np.arange(32768, dtype=np.uint32)
    z = (i * np.uint32(0x9E3779B1)) ^ np.uint32(seed)
    z ^= z >> np.uint32(15)
    z *= np.uint32(0x2C1B3C6D)
    z ^= z >> np.uint32(12)
    z *= np.uint32(0x297A2D39)
    z ^= z >> np.uint32(15)
    bits = (z & np.uint32(0x8000)) | ((np.uint32(14) + ((z >> np.uint32(10)) & np.uint32(1))) << np.uint32(10)) \
        | (z & np.uint32(0x3FF))
    return bits.astype(np.uint16).view(np.float16).astype(np.float64)


def fragment(h, start):
    """An operand fragment: lane l holds halves start + 8 l .. + 7; as the
    32 x 16 (A) or 16 x 32 (B, transposed here) matrix of a 32x32x16 product,
    lane l's element e sits at row l % 32, k = 8 (l // 32) + e."""
    f = h[start:start + 512].reshape(64, 8)
    return np.concatenate([f[:32], f[32:]], axis=1)  # [row][k]


def window_sums(h):
    """Per window w (steps with s % 8 == w): the sum of the 8 products'
    outputs and the sum of their absolute elementary products."""
    tot, mag = np.zeros(8), np.zeros(8)
    for w in range(8):
        base = 4096 * w
        A = [fragment(h, base + 512 * i) for i in range(4)]
        B = [fragment(h, base + 2048 + 512 * j) for j in range(2)]
        for a in A:
            for b in B:
                tot[w] += (a @ b.T).sum()
                mag[w] += (np.abs(a) @ np.abs(b).T).sum()
    return tot, mag


@pytest.mark.parametrize("seed,iters,wg", [(0x5EED, 1, 1), (7, 9, 3), (0x5EED, 64, 2), (123, 4096, 256)])
def test_mfma_ceiling_does_the_stated_products(q4lib, gpu, seed, iters, wg):
    import torch
    import bench
    L = bench.floor_lib()
    sink = torch.full((wg * 512,), float("nan"), dtype=torch.float32, device=gpu)
    rc = L.q4_mfma_ceiling(seed, iters, sink.data_ptr(), wg, torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    got = sink.cpu().numpy().astype(np.float64).reshape(wg * 8, 64)
    # every wave of every workgroup did the same work, lane by lane
    assert np.isfinite(got).all()
    assert (got == got[0]).all()
    tot, mag = window_sums(lds_values(seed))
    counts = np.array([(iters - w + 7) // 8 for w in range(8)], dtype=np.float64)  # steps per window
    expect = float(counts @ tot)
    bound = (iters + 128 + 16) * 2.0 ** -24 * float(counts @ mag)
    assert abs(got[0].sum() - expect) <= bound
