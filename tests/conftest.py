import os
import sys

import pytest
import torch  # noqa: F401  (load torch's HIP runtime before liboscar)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def golden():
    import json
    with open(os.path.join(ROOT, "tests", "golden", "pages_constants.json")) as f:
        return json.load(f)


def pytest_runtest_setup(item):
    if "gpu" in item.keywords:
        import torch
        if not torch.cuda.is_available():
            pytest.skip("needs a GPU")
