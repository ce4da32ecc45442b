import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# A test run may load another build of the library, e.g. the host-only build
# with AddressSanitizer and UndefinedBehaviorSanitizer that
# tests/test_sanitized_host.py makes; the binding then loads that file.
if os.environ.get("HSWA_TEST_LIBRARY"):
    from hybrid_sliding_window_hswa_amd import _capi
    _capi.LIB_PATH = os.environ["HSWA_TEST_LIBRARY"]


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running case")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def gpu():
    if not gpu_available():
        pytest.skip("no GPU visible")
    return True
