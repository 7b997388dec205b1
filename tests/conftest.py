import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)

# The library's testing aids (AD_NUM_SPLITS, AD_PARTIAL_KERNEL, AD_MFMA_TILE, AD_MFMA_ROWS,
# AD_FUSED_MERGE, AD_LPT) are read only while this switch is set; the tests set them per case.
os.environ["AD_TEST_KNOBS"] = "1"


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle

    return oracle.load()
