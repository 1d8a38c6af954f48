import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_finish(session):
    """When full-size GPU tests are selected, start generating their input tables in child
    processes now, before any test initialises the GPU in this process."""
    if any(item.get_closest_marker("gpu") is not None and "fullsize" in item.nodeid for item in session.items):
        import _tables
        _tables.start()


def pytest_sessionfinish(session, exitstatus):
    import sys as _sys
    mod = _sys.modules.get("_tables")
    if mod is not None:
        mod.stop()
