import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


@pytest.fixture(scope="session", autouse=True)
def _library_built():
    """Tests load the in-tree libmbert.so; build it only when nothing is built yet."""
    from pathlib import Path
    lib = Path(ROOT) / "transformer_encoder_amd" / "libmbert.so"
    if not lib.exists():
        from transformer_encoder_amd.build import build_library
        build_library()
    yield
