import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


_layers = {}


@pytest.fixture(scope="session")
def layer_cache():
    """Generated layers are reused across tests of one session."""
    import mpb_synth

    def get(cfg_id):
        if cfg_id not in _layers:
            _layers[cfg_id] = mpb_synth.make_layer(cfg_id)
        return _layers[cfg_id]
    return get
