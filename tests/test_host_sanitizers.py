"""The CPU code under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/sanitize/build_san.py builds the oracle and libvelox's host code
(argument checks and entry points, with launch stubs in place of the kernels)
with -fsanitize=address,undefined; the oracle tests and the C-ABI tests then
run in a child process against those builds (conftest.py swaps the library
paths when VELOX_TEST_LIBRARY / VELOX_TEST_ORACLE_LIBRARY are set).  Any
sanitizer report aborts the child, failing this test."""
import os
import subprocess
import sys

import pytest

from tests.sanitize.build_san import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def san_libs(tmp_path_factory):
    return build(str(tmp_path_factory.mktemp("san")))


def run_under_sanitizers(libs, tests):
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": libs["asan"],
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "VELOX_TEST_LIBRARY": libs["velox"],
        "VELOX_TEST_ORACLE_LIBRARY": libs["oracle"],
        "OMP_NUM_THREADS": "4",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider", "-m", "not gpu",
                        *tests], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail
    return r.stdout


def test_oracle_under_asan_ubsan(san_libs):
    out = run_under_sanitizers(san_libs, ["tests/test_oracle.py"])
    assert " passed" in out


def test_abi_validation_under_asan_ubsan(san_libs):
    out = run_under_sanitizers(san_libs, ["tests/test_abi.py"])
    assert " passed" in out
