import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle


def pytest_sessionfinish(session, exitstatus):
    """Writes the parity report (near-boundary counts per comparison) when SPECV_PARITY_REPORT
    names a file."""
    path = os.environ.get("SPECV_PARITY_REPORT")
    if not path:
        return
    try:
        import harness
    except ImportError:
        return
    if not harness.REPORT:
        return
    import json
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        json.dump(dict(exitstatus=int(exitstatus), entries=harness.REPORT), f, indent=1)
