import json
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Parity errors of the GPU path against the oracle, per named case: the GPU tests record them and
# the session writes them as JSON to the path in SWA_PARITY_REPORT (nothing when it is unset).
_PARITY = {}


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


@pytest.fixture(scope="session")
def parity():
    """record(name, abs_err): keep the max, mean and 99.9th percentile of |gpu - oracle| of a case
    (merged over calls with the same name: max of maxima, count-weighted mean, max of p99.9)."""
    def record(name, abs_err):
        e = np.asarray(abs_err, dtype=np.float64).ravel()
        if e.size == 0:
            return
        cur = {"max": float(e.max()), "mean": float(e.mean()), "p99.9": float(np.percentile(e, 99.9)),
               "elements": int(e.size)}
        old = _PARITY.get(name)
        if old is not None:
            n = old["elements"] + cur["elements"]
            cur = {"max": max(old["max"], cur["max"]),
                   "mean": (old["mean"] * old["elements"] + cur["mean"] * cur["elements"]) / n,
                   "p99.9": max(old["p99.9"], cur["p99.9"]), "elements": n}
        _PARITY[name] = cur
    return record


def pytest_sessionfinish(session, exitstatus):
    path = os.environ.get("SWA_PARITY_REPORT")
    if not _PARITY or not path:
        return
    try:
        os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
        with open(path, "w") as f:
            json.dump({"tolerance_max_abs": 2e-2, "cases": dict(sorted(_PARITY.items()))}, f, indent=1)
    except OSError:  # pragma: no cover
        pass
