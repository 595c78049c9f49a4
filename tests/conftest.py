import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; parity tests proper")
    config.addinivalue_line("markers", "slow: full-size workload checks")


@pytest.fixture(scope="session")
def q4lib():
    """The built libq4 (built here first if it is missing)."""
    import bit_block_quantized_q4_amd as q4
    if not q4.LIB_PATH.exists():
        from bit_block_quantized_q4_amd.build import build
        build()
    q4.lib()
    return q4


@pytest.fixture(scope="session")
def gpu(q4lib):
    """A usable GPU: fails (does not skip) when a gpu-marked test runs without one."""
    import torch
    assert torch.cuda.is_available(), "gpu-marked test needs a GPU"
    name = torch.cuda.get_device_properties(0).gcnArchName
    assert name.startswith("gfx950"), f"expected gfx950, found {name}"
    return torch.device("cuda:0")


@pytest.fixture(autouse=True)
def _announce(request):
    if request.node.get_closest_marker("gpu") is not None:
        sys.stdout.write(f"\n[gpu-test] {request.node.nodeid}\n")
        sys.stdout.flush()
    yield
