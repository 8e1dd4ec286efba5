import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-scale case (tens of GB of expert weights)")


def pytest_collection_modifyitems(config, items):
    # GPU tests fail loudly (not skip) when the library is missing; they are only
    # deselected by "-m 'not gpu'".
    pass
