import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


@pytest.fixture(autouse=True)
def _bounds_checked_build_clean(request):
    """With BDM_LIBRARY naming the bounds-checked build (libbdmoe_debug.so),
    every GPU test must leave that build's violation word clear."""
    yield
    if not os.environ.get("BDM_LIBRARY") or request.node.get_closest_marker("gpu") is None:
        return
    from block_diffusion_moe_amd import binding
    lib = binding._lib
    if lib is None or os.path.realpath(getattr(lib, "_name", "")) != \
            os.path.realpath(binding.DEBUG_LIB_PATH):
        return
    word = binding.bdm_debug_bounds()
    assert word == 0, f"bounds-check violations {word:#x} in the debug build"
