import os
import re
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


@pytest.hookimpl(hookwrapper=True)
def pytest_runtest_makereport(item, call):
    """A failing GPU parity test saves the cycle inputs of its workload as a
    replay (.npz) under $ET_REPLAY_DIR (default gpurun_out/replays), to be
    kept under tests/golden/replays/ and run again."""
    outcome = yield
    rep = outcome.get_result()
    if rep.when != "call" or not rep.failed:
        return
    cache = getattr(item.module, "_cache", None)
    params = getattr(getattr(item, "callspec", None), "params", {})
    name = params.get("name")
    if not cache or not name:
        return
    import replay
    out = os.environ.get("ET_REPLAY_DIR", os.path.join(ROOT, "gpurun_out", "replays"))
    for (n, tied), r in list(cache.items()):
        if n != name:
            continue
        os.makedirs(out, exist_ok=True)
        fn = re.sub(r"[^A-Za-z0-9_.-]+", "_", item.nodeid) + ("_tied" if tied else "") + ".npz"
        path = os.path.join(out, fn)
        replay.save(path, r["w"], r["inp"], note=f"failed: {item.nodeid}")
        rep.sections.append(("replay", f"inputs saved to {path}"))
