"""q4_gemm_noalloc (the GEMM whose workspace is the library's fixed
per-device scratch array) against q4_gemm on the same inputs: two calls in a
row, the second smaller, both needing scratch; outputs bit-identical to
q4_gemm's and within the oracle's tolerance."""

import numpy as np
import pytest

import oracle
import synth
from _gpu import assert_matmul_close, to_dev, to_dev_bf16, to_host

pytestmark = pytest.mark.gpu


def test_noalloc_matches_gemm_on_two_calls(q4lib, gpu):
    import torch
    # call 1: bf16 activations (staged as fp16 in the scratch) and a split-K
    # tail (fp32 partials after them); call 2: a smaller fp16 call with a tail
    cases = [(1030, 13200, 1024, "bf16"), (300, 11000, 1024, "f16")]
    for i, (m, n, k, xdt) in enumerate(cases):
        code = q4lib.Q4_BF16 if xdt == "bf16" else q4lib.Q4_F16
        need = q4lib.q4_gemm_workspace_size_dt(m, n, k, code)
        assert 0 < need <= q4lib.NOALLOC_SCRATCH_BYTES, (m, n, k, xdt, need)
        w = synth.random_weights(200 + i, n, k, "student_t")
        packed = oracle.quantize(w)
        pd = to_dev(packed, gpu)
        if xdt == "bf16":
            xb = synth.random_activations(210 + i, m, k, "bf16")
            xd, xref = to_dev_bf16(xb, gpu), oracle.widen_bf16(xb)
        else:
            xref = synth.random_activations(210 + i, m, k, "f16")
            xd = to_dev(xref, gpu)
        y_ref_gpu = to_host(q4lib.q4_gemm(xd, pd, y_dtype=torch.float32, n=n, k=k))
        y = torch.full((m, n), float("nan"), dtype=torch.float32, device=gpu)
        q4lib.q4_gemm_noalloc(xd, pd, y, n=n, k=k)
        got = to_host(y)
        assert np.array_equal(got.view(np.uint32), y_ref_gpu.view(np.uint32)), f"call {i}"
        assert_matmul_close(got, xref, packed, n, k, what=f"noalloc call {i} m{m} n{n} k{k}")
