import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def rng():
    import numpy as np
    return np.random.default_rng(20261202)


def pytest_terminal_summary(terminalreporter):
    """Per test, the largest max|err|/max|ref| that check() measured and its
    share of the tolerance; with QBLK_PARITY_LOG=<path> every comparison is
    also written there as JSON lines."""
    mod = sys.modules.get("gpu_util")
    log = getattr(mod, "PARITY_LOG", None) if mod else None
    if not log:
        return
    worst = {}
    for test, name, err, tol in log:
        r = err / tol if tol else float("inf")
        if test not in worst or r > worst[test][3]:
            worst[test] = (name, err, tol, r)
    terminalreporter.write_sep("-", f"parity: worst error per test ({len(log)} comparisons)")
    for test, (name, err, tol, r) in sorted(worst.items()):
        terminalreporter.write_line(f"{err:9.2e} / {tol:7.1e} = {r:5.3f}  {test}  [{name}]")
    path = os.environ.get("QBLK_PARITY_LOG")
    if path:
        import json
        with open(path, "w") as f:
            for test, name, err, tol in log:
                f.write(json.dumps({"test": test, "tensor": name, "err": err, "tol": tol}) + "\n")
