"""The benchmark's plain-read kernel (libq4floor) reads every byte once: the
XOR of its per-thread outputs equals the XOR of all the data's 32-bit words."""

import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,wg", [(16, 1), (4096, 3), (14745600, 256), (50135040, 2048)])
def test_read_floor_reads_every_word(q4lib, gpu, nbytes, wg):
    import torch
    import bench
    L = bench.floor_lib()
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(gpu)
    sink = torch.zeros(wg * 256, dtype=torch.int32, device=gpu)
    rc = L.q4_read_floor(buf.data_ptr(), nbytes, sink.data_ptr(), wg,
                         torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)
