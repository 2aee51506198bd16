import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


import pytest  # noqa: E402


@pytest.fixture
def ovr():
    """Set launch-shape overrides (slq_debug_override) for one test:
    ovr(MFMA_MIN_T=2, KS_GEMV=3); all are removed when the test ends."""
    import layer_sliced_quantized_amd as slq
    names = []

    def set_(**kw):
        for k, v in kw.items():
            slq.debug_override(k, int(v))
            names.append(k)

    yield set_
    for k in names:
        slq.debug_override(k, -1)
