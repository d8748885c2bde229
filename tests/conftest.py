import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle._load()
    return oracle


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def ne():
    """The HIP library binding; built in-tree first if nothing is built yet."""
    import causal_gqa_flashattention_attn_amd as ne_mod
    if not os.path.exists(ne_mod.library_path()):
        from causal_gqa_flashattention_attn_amd import _build
        _build.build()
    ne_mod.load()
    return ne_mod
