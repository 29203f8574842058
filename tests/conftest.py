import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Per-case parity figures (max-abs, rel-L2, score errors, ambiguous counts)
# collected by the GPU parity tests; printed in the terminal summary, so they
# survive output capture, and written as JSON to the file that the
# ISA_PARITY_RECORDS environment variable names, when it is set.
_RECORDS = []


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs through the C-ABI library")


@pytest.fixture
def parity_record():
    return _RECORDS.append


def pytest_terminal_summary(terminalreporter):
    if not _RECORDS:
        return
    terminalreporter.section("parity records")
    for rec in _RECORDS:
        terminalreporter.write_line(json.dumps(rec, sort_keys=True))
    path = os.environ.get("ISA_PARITY_RECORDS")
    if not path:
        return
    try:
        os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
        with open(path, "w") as f:
            json.dump(_RECORDS, f, indent=1, sort_keys=True)
    except OSError:
        pass
