import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


import pytest  # noqa: E402


@pytest.fixture(scope="session")
def built_lib():
    """Path of the in-tree libmagi_attn.so. In a container without a GPU
    (no /dev/kfd) a missing or stale library is rebuilt here with hipcc; on a
    GPU machine the library must have been built beforehand."""
    from block_causal_attention_flash_amd import build as b
    if b.is_stale():
        if os.path.exists("/dev/kfd"):
            if not os.path.exists(b.LIB):
                pytest.fail(f"{b.LIB} is missing; build it before running the GPU tests")
        else:
            b.build()
    return b.LIB
