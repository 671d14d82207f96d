import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path through the C ABI")


def _ensure_built():
    """Build the CPU-side helper libraries if nothing is built yet (gcc, seconds)."""
    import importlib
    for mod, lib in (("synth.build", "synth/libsynth.so"), ("oracle.build", "oracle/liboracle.so")):
        if not os.path.exists(os.path.join(ROOT, lib)):
            importlib.import_module(mod).build()


_ensure_built()


@pytest.fixture(scope="session")
def root():
    return ROOT
