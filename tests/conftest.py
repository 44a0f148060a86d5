import os
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running (full-size configurations)")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle

    if not (Path(oracle.__file__).parent / "liboracle.so").exists():
        oracle.build(force=True)
    return oracle


def gpu_available() -> bool:
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


@pytest.fixture(scope="session")
def dsa_gpu():
    """The product binding on cuda:0; fails loudly if the HIP library is missing."""
    if not gpu_available():
        pytest.fail("GPU test collected without a GPU (run with -m 'not gpu' on CPU hosts)")
    import dsa_sparse_attention_indexer_amd as dsa

    dsa.load_library()  # raises if libdsa.so is absent
    return dsa


def pytest_report_header(config):
    return f"cwd={os.getcwd()}"
