import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


LIB = os.path.join(ROOT, "bit_quantized_matmul_col_amd", "libllmint8.so")
RESOURCES = os.path.join(ROOT, "bit_quantized_matmul_col_amd", "libllmint8.kernels.json")


@pytest.fixture(scope="session")
def built_library():
    """The HIP library and its kernel-resource record, built here (hipcc
    cross-compiles gfx950 without a GPU) when they are missing: the tests that
    need them fail on a broken build instead of skipping."""
    if not (os.path.exists(LIB) and os.path.exists(RESOURCES)):
        from bit_quantized_matmul_col_amd import build
        build.build()
    assert os.path.exists(LIB) and os.path.exists(RESOURCES)
    return LIB
