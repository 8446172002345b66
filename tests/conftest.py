import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size parity case (minutes of CPU oracle work)")


@pytest.fixture(scope="session")
def fa():
    """The GPU binding; loading it fails loudly if the library is missing."""
    import exact_tiled_attention_17_amd as fa_mod
    fa_mod.load()
    return fa_mod
