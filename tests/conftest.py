import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


# The host-sanitizer test runs the ABI tests again in a child process against
# a CPU-only ASan/UBSan build of the library's host code (tests/sanitizer);
# this variable points the binding at that build for the child only.
_SANITIZER_LIB = os.environ.get("EEA_SANITIZER_LIB")
if _SANITIZER_LIB:
    import efficient_exact_attention_amd as _ea
    _ea._LIB_PATH = _SANITIZER_LIB
