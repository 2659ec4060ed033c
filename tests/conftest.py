import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size case (minutes)")


def pytest_collection_modifyitems(config, items):
    # GPU tests need a device; skip them loudly where there is none.
    import torch
    if torch.cuda.is_available():
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


@pytest.hookimpl(hookwrapper=True)
def pytest_runtest_makereport(item, call):
    # A HIP runtime error (memory fault, illegal address) poisons the device
    # for the rest of the process: stop the whole session at the first one
    # instead of letting later tests run on a faulted GPU.
    outcome = yield
    rep = outcome.get_result()
    if rep.failed and call.excinfo is not None:
        text = str(call.excinfo.value)
        if "HIP error" in text or "hipError" in text or "illegal memory" in text:
            pytest.exit(f"HIP runtime error in {item.nodeid}: {text.splitlines()[0]}",
                        returncode=3)
