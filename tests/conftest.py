"""Shared test setup: repository root on sys.path, the `gpu` marker, and the
build of the oracle / product library when none is present."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Build what is missing (the oracle and the library are compiled in-tree; a
# machine that receives the tree with its built files does not rebuild them).
from oracle import build as _oracle_build  # noqa: E402
from decode_attention_paged_slot_amd import build as _pda_build  # noqa: E402

_oracle_build.ensure_built()
if not os.path.exists(_pda_build.LIB):
    _pda_build.build()


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def _gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if any("gpu" in item.keywords for item in items) and not _gpu_available():
        skip = pytest.mark.skip(reason="no GPU visible")
        for item in items:
            if "gpu" in item.keywords:
                item.add_marker(skip)
