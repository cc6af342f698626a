import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line(
        "markers", "slow: long CPU-side oracle work")


# RECSA_TEST_ROTATED_KEYS=0 runs every test on trees without the rotated-key
# copy Kr (the kernels rotate raw key rows), unless a test asks for it.
if os.environ.get("RECSA_TEST_ROTATED_KEYS") == "0":
    from long_context_kv_amd import recsa as _R

    _allocate = _R.Tree.allocate

    def _allocate_without_kr(*args, **kwargs):
        kwargs.setdefault("rotated_keys", False)
        return _allocate(*args, **kwargs)

    _R.Tree.allocate = staticmethod(_allocate_without_kr)
