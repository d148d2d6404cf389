import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running check (minutes)")


def pytest_collection_modifyitems(config, items):
    # gpu tests cannot run without a device; mark them skipped rather than failing
    # when someone runs the whole suite on a CPU-only machine.
    if os.environ.get("ORACLE_MUTANT_LIB") or os.environ.get("ORACLE_MUTANT_PY"):
        have_gpu = False          # a mutation run checks the CPU pins only
    else:
        try:
            import torch
            have_gpu = torch.cuda.is_available()
        except Exception:  # pragma: no cover
            have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)
