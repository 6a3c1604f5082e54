import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")
    # FA_TEST_LIBRARY points the binding at another build of the library (the
    # host-sanitized one); it must be loaded before any test module reads
    # fa.LIB_PATH or calls fa.load_library().
    alt = os.environ.get("FA_TEST_LIBRARY")
    if alt:
        from exact_attention_122_amd import fa
        fa.LIB_PATH = alt
        fa.load_library(alt)
        sys.__stderr__.write(f"[library] {alt}\n")
        sys.__stderr__.flush()


def pytest_collection_modifyitems(config, items):
    # GPU tests only make sense with a device; skip them loudly otherwise.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_runtest_logstart(nodeid, location):
    # name the case before any GPU work starts, so a run that dies still says where
    if "gpu" in nodeid:
        sys.__stderr__.write(f"[start] {nodeid}\n")
        sys.__stderr__.flush()
