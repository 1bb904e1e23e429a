import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (HIP device)")
    config.addinivalue_line("markers", "slow: long CPU test")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    import oracle
    oracle.build(force=False)
    yield


def pytest_terminal_summary(terminalreporter):
    """Near-tie events of the GPU draft-step replays (one per sequence and
    step whose frontier differs from the oracle's only inside a near tie)."""
    gu = sys.modules.get("gpu_util")
    if gu is None or not getattr(gu, "NEAR_TIES", None):
        return
    terminalreporter.write_sep("-", "near-tie events (GPU replay vs oracle)")
    for name, (ev, steps) in sorted(gu.NEAR_TIES.items()):
        terminalreporter.write_line(f"{name}: {ev} event(s) in {steps} sequence-steps")
