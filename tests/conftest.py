import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def read_golden(name):
    """Non-comment lines of a golden fixture file."""
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.lstrip().startswith("#")]


@pytest.fixture
def force():
    """force(key, value) sets one of the library's tuning overrides for this
    test; every key it touched is restored to automatic (-1) afterwards."""
    import block_scaled_fp4_gemm_amd as bg

    touched = []

    def set_(key, value):
        touched.append(key)
        bg.tune_set(key, value)

    yield set_
    for key in touched:
        bg.tune_set(key, -1)
