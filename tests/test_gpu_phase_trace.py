"""The measurement build libq4trace.so (tile GEMV with per-phase clock stamps,
used only by `bench.py --phase-trace`) computes exactly what libq4.so does and
records one ordered set of stamps per computing wave."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("m,n,k", [(10, 30000, 1024), (10, 5120, 2048), (16, 4096, 1536)])
def test_trace_build_matches_the_product_and_records_phases(q4lib, gpu, m, n, k):
    import torch
    import bench
    L = bench.trace_lib()
    gen = torch.Generator(device=gpu)
    gen.manual_seed(n + k)
    w = torch.randn((n, k), device=gpu, generator=gen) * 0.02
    packed = q4lib.q4_quantize(w)
    x = torch.randn((m, k), device=gpu, generator=gen).half()
    y_prod = q4lib.q4_gemv(x, packed, y_dtype=torch.float32)
    stamps = torch.zeros(((n + 15) // 16 + 1) * 8 * bench.PHASE_SLOTS, dtype=torch.int64, device=gpu)
    saved = q4lib._LIB
    try:
        q4lib._LIB = L
        assert L.q4_phase_trace_set(stamps.data_ptr()) == 0
        y_trace = q4lib.q4_gemv(x, packed, y_dtype=torch.float32)
        torch.cuda.synchronize()
        assert L.q4_phase_trace_set(None) == 0
    finally:
        q4lib._LIB = saved
    assert torch.equal(y_prod, y_trace)
    T = stamps.view(-1, 8, bench.PHASE_SLOTS).cpu().numpy()
    ran = T[:, 0, 0] > 0
    assert ran.any()
    d = bench.phase_summary(T)
    assert d["phases"] >= 1
    p = d["phases"]
    for t in T[ran]:
        bars = t[0, 1:1 + p]
        assert np.all(np.diff(bars) > 0)                     # barriers in order
        assert np.all(t[:, 32:32 + p] >= bars)               # products after their barrier
        assert t[0, 63] >= t[:, 32 + p - 1].max()              # exit after every wave's last phase
        assert t[0, 62] > t[0, 31] > 0                         # constant-clock stamps at entry and exit
    assert 100.0 < d["sclk_mhz"] < 3000.0                      # a shader clock MI355X can run at
