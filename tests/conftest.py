import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def cb2():
    """The 2-bit codebook (m=4, 256 codes) the oracle builds from the
    workloads' 65536 seed-0 samples, read from the stored golden file."""
    from tests.golden import load_codebook
    return load_codebook(4)


@pytest.fixture(scope="session")
def cb1():
    from tests.golden import load_codebook
    return load_codebook(8)
