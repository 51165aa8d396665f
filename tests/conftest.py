import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


# The host-only sanitizer build of the C ABI is tested by running the CPU
# ABI tests in a child process against that library (test_sanitizers_cpu).
if os.environ.get("KVQ_TEST_LIBRARY"):
    from int2_rotated_kv_amd import kvq as _kvq
    _kvq._LIB_PATH = os.environ["KVQ_TEST_LIBRARY"]
