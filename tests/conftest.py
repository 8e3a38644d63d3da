import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
for p in (ROOT, os.path.dirname(os.path.abspath(__file__))):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; calls the HIP library")


import importlib.util

import pytest


def _build_module():
    """Load context_parallelism_cp_amd/build.py without importing the package
    (whose import needs the library to exist already)."""
    path = os.path.join(ROOT, "context_parallelism_cp_amd", "build.py")
    spec = importlib.util.spec_from_file_location("_cpattn_build", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="session", autouse=True)
def _libraries_built():
    """Build the C oracle and libcpattn.so only when nothing is built yet."""
    from oracle import native
    native._load()
    if not os.path.exists(os.path.join(ROOT, "context_parallelism_cp_amd", "libcpattn.so")):
        _build_module().build()
