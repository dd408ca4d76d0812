import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def lib():
    """The C-ABI library through its Python binding (fails loudly if it is not built)."""
    from speculative_decoding_verify_02_amd import binding
    return binding.load()


def pytest_sessionfinish(session, exitstatus):
    """With PARITY_MARGINS_OUT set, write every parity check's worst errors (JSON)."""
    path = os.environ.get("PARITY_MARGINS_OUT")
    mod = sys.modules.get("test_verify_attn_gpu")
    if not path or mod is None or not getattr(mod, "MARGINS", None):
        return
    import json
    with open(path, "w") as f:
        json.dump(mod.MARGINS, f, indent=0)
