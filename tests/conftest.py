import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def pytest_collection_modifyitems(config, items):
    """A GPU run without the built library is an error, not a run of skipped tests.

    The GPU test modules skip themselves when the library cannot be imported
    (so the CPU suite can collect them on a machine without a build); when a
    GPU test is selected and a GPU is present, the import must succeed.
    """
    if not any(item.get_closest_marker("gpu") for item in items):
        return
    import torch
    if not torch.cuda.is_available():
        return
    try:
        import mxfp4_weight_mixture_amd  # noqa: F401
    except ImportError as e:
        raise pytest.UsageError(f"GPU tests selected but the HIP library does not load: {e}")
