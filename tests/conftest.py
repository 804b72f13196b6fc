import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libc3.so")


@pytest.fixture(scope="session")
def orc():
    """The CPU oracle (built with gcc on first use if liboracle.so is missing)."""
    import oracle

    oracle.lib()
    return oracle


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Name every GPU case on stdout (flushed) before it touches the device."""
    if request.node.get_closest_marker("gpu") is not None:
        print(f"\n[gpu-case] {request.node.nodeid}", flush=True)
    yield


_GPU_USED = []


@pytest.fixture
def host_only():
    """For tests that start child processes (gcc, bench.py): skipped once this process has
    initialised the GPU, since a child forked after that must not exec another program."""
    t = sys.modules.get("torch")
    if _GPU_USED or (t is not None and t.cuda.is_initialized()):
        pytest.skip("this process has initialised the GPU; no child processes are started")


@pytest.fixture(scope="session")
def c3gpu():
    """libc3 bound to cuda:0. GPU tests fail (never skip) when no GPU is visible."""
    import torch

    _GPU_USED.append(True)

    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    from concurrent_gemm_dma_amd import _c3

    _c3.c3_init(0)
    yield _c3
    torch.cuda.synchronize()
    _c3.c3_finalize()
