import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


_POISONED = []


@pytest.fixture(scope="session")
def gpu_lib():
    """The built HIP library through its Python binding (GPU tests only),
    with every output it allocates NaN-filled and followed by a canary tail
    (tests/gpu_util.PoisonedLib); the tails are checked after each test."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import subquadratic_attention_amd as sqa
    from tests.gpu_util import PoisonedLib

    sqa.load_library()
    lib = PoisonedLib(sqa)
    _POISONED.append(lib)
    return lib


@pytest.fixture(autouse=True)
def _output_canaries():
    """After every test: no kernel wrote past the end of an output buffer."""
    yield
    for lib in _POISONED:
        lib.check_canaries()
