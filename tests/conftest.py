import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _ensure_cpu_libs():
    """Build the C generator and the C oracle if they are missing (gcc, seconds)."""
    import oracle
    import synth

    if not os.path.exists(oracle.lib_path()):
        oracle.build()
    if not os.path.exists(synth.lib_path()):
        synth.build()


_ensure_cpu_libs()


@pytest.fixture(scope="session")
def rng_seed():
    return 1234
