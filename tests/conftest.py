import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.fixture(scope="session")
def consts():
    return load_golden("format_constants.json")


def pytest_runtest_logstart(nodeid, location):
    # name the case on the unbuffered stream before it touches the GPU, so a
    # run that ends abruptly still shows which test was running
    if "gpu" in nodeid or "smoke" in nodeid:
        sys.__stderr__.write(f"[case] {nodeid}\n")
        sys.__stderr__.flush()


def pytest_collection_modifyitems(config, items):
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible (run on an MI355X box)")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
