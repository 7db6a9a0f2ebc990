import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _have_gpu() -> bool:
    try:
        import torch
        return torch.cuda.is_available() and torch.cuda.device_count() > 0
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _have_gpu():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


@pytest.fixture
def tune():
    """tune(knob, value): force a kernel choice through macaq_set_tuning for
    the rest of the test; every knob touched is set back afterwards."""
    import mxfp4_w4a4_quantized_channel_amd as mx
    before = {}

    def set_knob(knob, value):
        prev = mx.set_tuning(knob, value)
        before.setdefault(knob, prev)

    yield set_knob
    for knob, value in before.items():
        mx.set_tuning(knob, value)
