import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Achieved parity figures (max errors, oracle self-divergence, flip and
# near-tie counts) recorded by the GPU tests.  They are printed in the terminal
# summary, which pytest shows under -q too, and written as JSON to the path in
# DSTILL_PARITY_RECORD when that variable is set.
_RECORD: dict = {}


@pytest.fixture
def parity_record(request):
    def rec(**values):
        entry = _RECORD.setdefault(request.node.nodeid.split("::", 1)[-1], {})
        for k, v in values.items():
            entry[k] = float(v) if isinstance(v, float) else v
    return rec


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


def pytest_collection_modifyitems(config, items):
    # GPU tests cannot run without a device: skip them with a reason rather
    # than failing when the marker filter was not given.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


def pytest_terminal_summary(terminalreporter):
    if not _RECORD:
        return
    tr = terminalreporter
    tr.section("parity record (achieved GPU-oracle figures)")
    for name, vals in _RECORD.items():
        parts = []
        for k, v in vals.items():
            parts.append(f"{k}={v:.3e}" if isinstance(v, float) else f"{k}={v}")
        tr.write_line(f"{name}: " + ", ".join(parts))
    path = os.environ.get("DSTILL_PARITY_RECORD")
    if path:
        with open(path, "w") as f:
            json.dump(_RECORD, f, indent=1, sort_keys=True)
