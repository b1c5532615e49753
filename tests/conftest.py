import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU oracle work")


@pytest.fixture(scope="session")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def pytest_sessionfinish(session, exitstatus):
    """With Q3_PARITY_LOG set, write every parity comparison of the run (test, tensor,
    element count, max-abs and mean-relative error with their bars) to that JSON file."""
    path = os.environ.get("Q3_PARITY_LOG")
    if not path:
        return
    try:
        import q3_testutil
    except ImportError:
        return
    import json
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        json.dump(q3_testutil.RECORDS, f, indent=1)
