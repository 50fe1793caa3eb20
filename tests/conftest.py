import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests fail loudly (not skip) when the HIP library is missing on a machine with a GPU; on a host
    # without a GPU they are only deselected by -m "not gpu".
    pass


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


@pytest.fixture
def golden():
    return golden_rows
