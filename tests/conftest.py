import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    """Build the CPU oracle once if it has not been built yet."""
    import oracle
    if not os.path.exists(os.path.join(ROOT, "oracle", "liblcd_oracle.so")):
        oracle.build()
    yield


@pytest.fixture(scope="session")
def gpu():
    """Fail loudly (never skip) when a GPU test runs without a usable GPU or
    without the built HIP library."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but torch.cuda.is_available() is False")
    import context_lookup_drafting_amd as lcd
    lcd.load()  # raises if liblcd.so is missing or does not load
    return torch.device("cuda:0")
