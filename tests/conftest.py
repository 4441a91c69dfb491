import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # The host-sanitized test runs the bookkeeping fuzzers in a child process
    # against the sanitized build of the library, named here; nothing else
    # sets this.
    lib = os.environ.get("PA_TEST_SANITIZED_LIBRARY")
    if lib:
        from paged_kv_cache_block_amd import abi
        abi.LIB_PATH = lib
