import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


# A host-side build of the C ABI under sanitizers (tests/test_host_sanitizers.py)
# replaces the library for the child process that runs the ABI test modules.
if os.environ.get("KIVI_HOST_SANITIZED_LIB"):
    import kv_cache_quantization_codec_amd.binding as _binding

    _binding.LIB_PATH = os.environ["KIVI_HOST_SANITIZED_LIB"]


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")
