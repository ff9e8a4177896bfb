import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running (full-size workloads)")


def pytest_sessionfinish(session, exitstatus):
    """With PA_PARITY_REPORT set, write the largest max-abs error recorded per
    named workload (tests.gpu_helpers.record_max_abs) to that JSON file."""
    path = os.environ.get("PA_PARITY_REPORT")
    helpers = sys.modules.get("tests.gpu_helpers")
    if not path or helpers is None or not helpers.MAX_ABS:
        return
    import json
    d = os.path.dirname(path)
    if d:
        os.makedirs(d, exist_ok=True)
    with open(path, "w") as f:
        json.dump({k: float(v) for k, v in sorted(helpers.MAX_ABS.items())}, f, indent=1)
        f.write("\n")
