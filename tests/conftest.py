import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.dirname(os.path.abspath(__file__))
for p in (TESTS, ROOT):
    if p not in sys.path:
        sys.path.insert(0, p)

# The sanitized host-logic build of the C ABI (tests/test_abi_sanitized.py) runs the
# ABI tests in a child process against that library instead of libmoe.so.
_HOST_LIB = os.environ.get("MOE_TEST_HOST_LIB")
if _HOST_LIB:
    from sparse_mixture_experts_13_amd import _lib as _moe_lib
    _moe_lib.LIB_PATH = _HOST_LIB


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (minutes of host work)")
