import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle.default()


def pytest_sessionfinish(session, exitstatus):
    # The f32 bar's headroom per GPU test (largest |y - y_oracle| / T), when
    # asked for.
    out = os.environ.get("XQ_HEADROOM_OUT")
    mod = sys.modules.get("test_gpu_parity")
    if not out or mod is None or not getattr(mod, "HEADROOM", None):
        return
    import json
    with open(out, "w") as f:
        json.dump(dict(sorted(mod.HEADROOM.items())), f, indent=1)
