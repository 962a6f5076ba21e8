import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; run on the GPU box")
    config.addinivalue_line("markers", "slow: large-shape CPU check")


def _swap_libraries():
    """Host-sanitizer runs (test_host_sanitizers.py) point the loaders at the
    sanitized builds of the host code and the oracle."""
    lib = os.environ.get("VELOX_TEST_LIBRARY")
    if lib:
        import geometry_routed_block_velox_amd as velox
        velox.library_path = lib
    olib = os.environ.get("VELOX_TEST_ORACLE_LIBRARY")
    if olib:
        from oracle import velox_oracle
        velox_oracle._LIB_PATH = olib


_swap_libraries()
