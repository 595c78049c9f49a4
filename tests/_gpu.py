"""Helpers for the GPU parity tests: host <-> device copies and oracle checks."""

import numpy as np

import oracle


def to_dev(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def to_dev_bf16(bits, dev):
    """uint16 bfloat16 patterns -> a torch.bfloat16 device tensor (same bits)."""
    import torch
    a = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(a).view(torch.bfloat16).to(dev)


def to_host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_matmul_close(g, x, packed_host, n, k, cols=None, what=""):
    """Every GPU output within 1e-3 * sum|w*x| + 1e-6 of the oracle."""
    y, S = oracle.matmul_ref(x, packed_host, n, k, cols=cols)
    ok, worst, idx = oracle.check(g, y, S)
    assert ok, (f"{what}: worst |gpu-oracle|/bound = {worst:.3g} at {idx}: "
                f"gpu={np.asarray(g)[idx]!r} oracle={y[idx]!r} S={S[idx]!r}")
    return worst


def sample_rows(m, count, seed):
    """Sorted row sample that always includes the first and last rows."""
    rng = np.random.default_rng(seed)
    if m <= count:
        return np.arange(m)
    pick = set(rng.choice(m, size=count - 2, replace=False).tolist()) | {0, m - 1}
    return np.array(sorted(pick))


_WEIGHT_CACHE = {}


def workload_weights_cached(wl, lin):
    """Host weights of a workload linear, generated once per test session."""
    key = (wl.wid, lin.tensor_id)
    if key not in _WEIGHT_CACHE:
        import synth
        _WEIGHT_CACHE[key] = synth.workload_weights(wl, lin)
    return _WEIGHT_CACHE[key]
