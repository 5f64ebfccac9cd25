import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


import pytest  # noqa: E402


@pytest.fixture(scope="module")
def fga():
    """The binding, with fresh NaN-filled outputs and workspaces framed by guard bands on
    every call (tests/guarded.py)."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import full_gqa_attention_amd as m
    from guarded import Guarded
    return Guarded(m)
