import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")


def pytest_runtest_setup(item):
    # A GPU test that starts on a machine without a GPU is an error of the run, not a skip:
    # a skip would let the GPU suite look green without the native code having run.
    # Select the CPU suite with -m "not gpu".
    if "gpu" in item.keywords:
        import torch
        if not torch.cuda.is_available():
            pytest.fail("gpu-marked test started without a visible GPU (run the CPU suite with -m 'not gpu')")
