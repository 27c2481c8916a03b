import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


# The host-sanitizer test runs the ABI tests in a child process against the sanitized build of the library.
if os.environ.get("QSA_TEST_LIB"):
    import sparse_top_attention_amd as _qsa
    _qsa.LIB_PATH = os.environ["QSA_TEST_LIB"]


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
