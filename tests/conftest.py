import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def golden():
    import json
    with open(os.path.join(ROOT, "tests", "golden", "worked_examples.json")) as f:
        return json.load(f)


@pytest.fixture(scope="session")
def t1_golden():
    import json
    with open(os.path.join(ROOT, "tests", "golden", "t1_layout.json")) as f:
        return json.load(f)


@pytest.fixture(scope="session")
def lut_golden():
    import json
    with open(os.path.join(ROOT, "tests", "golden", "lut_table.json")) as f:
        return json.load(f)


@pytest.fixture(scope="session")
def prefill_golden():
    import json
    with open(os.path.join(ROOT, "tests", "golden", "prefill_layout.json")) as f:
        return json.load(f)
