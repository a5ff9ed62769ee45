import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_collection_modifyitems(config, items):
    # A gpu-marked test cannot run without a visible GPU: skip it with the reason
    # instead of failing at the first HIP call.
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


@pytest.fixture
def options():
    """Sets the library's process-wide path options (jfa_set_option) for one
    test: options(name, value); every option returns to the library's
    choice afterwards."""
    from jagged_attention_ads_amd import jfa
    yield jfa.set_option
    for name in jfa.OPTIONS:
        jfa.set_option(name, None)
