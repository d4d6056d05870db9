import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-geometry oracle runs (minutes of CPU)")


@pytest.fixture(scope="session")
def slice3():
    """The three-layer slice (conv, sliding, full) at real width, q4 g64, seeded."""
    from attention_decoder_amd import synth
    cfg = synth.slice3_config()
    blob = synth.cached_blob(cfg, seed=0)
    return cfg, blob


@pytest.fixture(scope="session")
def slice3_oracle(slice3):
    from oracle import Oracle
    cfg, blob = slice3
    return Oracle(cfg, blob)
