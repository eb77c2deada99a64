import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running GPU case (full-size workloads)")


import pytest  # noqa: E402


@pytest.fixture(autouse=True)
def _default_tuning():
    """Every test starts from the library's own launch-shape choices: tuning
    overrides a test sets are undone after it."""
    yield
    kda = sys.modules.get("gated_delta_rule_diag_amd.kda")
    if kda is not None and kda._lib is not None:
        kda.set_tuning()
