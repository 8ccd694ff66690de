import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")


def pytest_collection_modifyitems(config, items):
    gpu_items = [it for it in items if it.get_closest_marker("gpu")]
    if not gpu_items:
        return
    import torch
    if not torch.cuda.is_available():
        skip = pytest.mark.skip(reason="no GPU visible")
        for it in gpu_items:
            it.add_marker(skip)
        return
    # the library is built in-tree beforehand; build only if nothing is there
    from fp4_kv_cache_e2m1_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from fp4_kv_cache_e2m1_amd import build_lib
        build_lib.build()


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")
