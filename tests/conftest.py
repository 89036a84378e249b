import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size parity case (seconds of oracle work)")


@pytest.fixture(scope="session")
def gpu():
    """The loaded HIP binding; skips nothing -- a GPU test without a GPU is a failure."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("gpu-marked test run without a visible GPU")
    from gemm_q8_amd import gq8
    return gq8


def pytest_sessionfinish(session, exitstatus):
    """With GQ8_PARITY_REPORT=<path>, write every parity check's worst ratios (tests/helpers.py)
    as JSON lines."""
    path = os.environ.get("GQ8_PARITY_REPORT")
    if not path:
        return
    import json
    try:
        from tests.helpers import RECORDS
    except ImportError:
        return
    with open(path, "w") as f:
        for r in RECORDS:
            f.write(json.dumps(r) + "\n")
