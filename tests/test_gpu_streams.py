"""The library keeps no state between calls: launches on two streams at once
(each with its own outputs and GEMM workspace) give exactly the results of the
same calls run one after another."""

import numpy as np
import pytest

import oracle
import synth
from _gpu import to_dev, to_host

pytestmark = pytest.mark.gpu


def test_two_streams_match_sequential(q4lib, gpu):
    import torch
    n, k = 5120, 5120
    w = to_dev(synth.random_weights(61, n, k, "student_t"), gpu)
    packed = q4lib.q4_quantize(w)
    xs = {m: to_dev(synth.random_activations(62 + m, m, k, "f16"), gpu) for m in (1, 4, 10, 16)}
    xg = to_dev(synth.random_activations(70, 384, k, "f16"), gpu)
    torch.cuda.synchronize()
    # sequential reference on the default stream
    ref_v = {m: to_host(q4lib.q4_gemv(xs[m], packed, y_dtype=torch.float32)) for m in xs}
    ref_g = to_host(q4lib.q4_gemm(xg, packed, y_dtype=torch.float32))
    ref_q = to_host(packed)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs_v = {m: torch.empty((m, n), dtype=torch.float32, device=gpu) for m in xs}
    out_g = torch.empty((384, n), dtype=torch.float32, device=gpu)
    out_q = torch.empty_like(packed)
    ws = torch.empty(max(q4lib.q4_gemm_workspace_size(384, n, k), 1), dtype=torch.uint8, device=gpu)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in list(outs_v.values()) + [out_g]:
            t.fill_(float("nan"))
        out_q.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            for _ in range(4):
                for m in xs:
                    q4lib.q4_gemv(xs[m], packed, y=outs_v[m], stream=s1)
            q4lib.q4_quantize(w, packed=out_q, stream=s1)
        with torch.cuda.stream(s2):
            q4lib.q4_gemm(xg, packed, y=out_g, workspace=ws, stream=s2)
        torch.cuda.synchronize()
        for m in xs:
            assert np.array_equal(to_host(outs_v[m]).view(np.uint32), ref_v[m].view(np.uint32)), (rep, m)
        assert np.array_equal(to_host(out_g).view(np.uint32), ref_g.view(np.uint32)), rep
        assert np.array_equal(to_host(out_q), ref_q), rep
    # and the reference itself is right (sampled columns)
    cols = np.arange(0, n, 97)
    y, S = oracle.matmul_ref(to_host(xs[10]), ref_q, n, k, cols=cols)
    assert oracle.check(ref_v[10][:, cols], y, S)[0]
