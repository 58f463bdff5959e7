import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
for _p in (ROOT, os.path.join(ROOT, "tests")):
    if _p not in sys.path:
        sys.path.insert(0, _p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a real MI355X (gfx950) and the built HIP library")


@pytest.fixture(scope="session")
def golden():
    import json

    gdir = os.path.join(ROOT, "tests", "golden")

    def load(name):
        with open(os.path.join(gdir, name)) as f:
            return json.load(f)

    return load
