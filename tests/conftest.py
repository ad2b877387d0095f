import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def lib():
    """The ctypes-loaded libfa.so (built in-tree first if it is missing)."""
    import exact_attention_83_amd as fa
    if not os.path.exists(fa.LIB_PATH):
        from exact_attention_83_amd import build
        build.build()
    return fa.load()


@pytest.fixture(scope="session")
def fa_gpu(lib):
    """The binding module, on a host whose GPU is visible; fails loudly if not."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run on a host without a visible GPU")
    import exact_attention_83_amd as fa
    return fa


def say(msg):
    """Name the case about to run on the GPU (flushed, so a crash keeps it)."""
    print(f"[gpu-case] {msg}", flush=True)
