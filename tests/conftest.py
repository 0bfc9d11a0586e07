import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_sessionfinish(session, exitstatus):
    """With MSS_PARITY_MARGINS=<file>, write the recorded worst error / limit ratios (JSON)."""
    path = os.environ.get("MSS_PARITY_MARGINS")
    if not path:
        return
    try:
        from tests.gpu_helpers import MARGINS
    except ImportError:
        return
    if MARGINS:
        import json
        with open(path, "w") as f:
            json.dump(dict(sorted(MARGINS.items())), f, indent=1)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle.build(force=False)
    return oracle


@pytest.fixture
def plan():
    """Fixes the library's plans (mss_set_plan_overrides) for one test and restores the automatic
    plans afterwards, also when the test fails."""
    import selective_state_space_06_amd as mss
    yield lambda **kw: mss.set_plan_overrides(**kw)
    mss.set_plan_overrides()
