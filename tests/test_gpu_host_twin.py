"""One weight copy, two backends: the bytes the GPU quantiser writes, read
unchanged by the GPU GEMV and by the host-CPU twin, both within tolerance of
the oracle (full-size decode workloads, sampled output features)."""

import numpy as np
import pytest

import synth
from _gpu import assert_matmul_close, to_dev, to_host, workload_weights_cached

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wid", [2, 3])
def test_gpu_bytes_on_both_backends(q4lib, gpu, wid):
    import torch
    from bit_block_quantized_q4_amd.host import q4_host_gemv
    wl = synth.WORKLOADS[wid]
    lin = wl.linears[0]
    w = workload_weights_cached(wl, lin)
    packed_d = q4lib.q4_quantize(to_dev(w, gpu))
    packed = to_host(packed_d)
    del w
    rng = np.random.default_rng(wid)
    cols = np.unique(np.concatenate([rng.choice(lin.n, size=512, replace=False), [0, lin.n - 1]]))
    for m in wl.ms:
        x = synth.workload_activations(wl, lin.k, m)
        yg = to_host(q4lib.q4_gemv(to_dev(x, gpu), packed_d, y_dtype=torch.float32))
        yh = q4_host_gemv(x, packed, y_dtype=np.float32)
        assert_matmul_close(yg[:, cols], x, packed, lin.n, lin.k, cols=cols, what=f"gpu m{m}")
        assert_matmul_close(yh[:, cols], x, packed, lin.n, lin.k, cols=cols, what=f"host m{m}")
