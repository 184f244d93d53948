import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _ensure_built():
    """Build the HIP library in-tree if it is not there yet (an existing build
    is used as is)."""
    lib = os.path.join(ROOT, "fp4_quantized_prep_amd", "libiqprep.so")
    if not os.path.exists(lib):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_iqp_build", os.path.join(ROOT, "fp4_quantized_prep_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()


def pytest_configure(config):
    _ensure_built()
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


@pytest.fixture(scope="session")
def gpu_lib():
    """The product binding, with the HIP library loaded on a GPU device."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp4_quantized_prep_amd as iqp
    return iqp
