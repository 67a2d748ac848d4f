import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import __graft_entry__  # noqa: E402

# Build whatever native part is missing (nothing is rebuilt if present).
__graft_entry__.ensure_built()


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs a gfx950 (MI355X) device; runs the HIP library")
