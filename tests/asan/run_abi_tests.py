"""Run the host-only C-ABI tests (tests/test_abi.py) against another build of the library.

Usage: python tests/asan/run_abi_tests.py <path to library> [pytest args...].  The binding is pointed
at the given library before the tests import it; used for the sanitizer build of the host layer."""

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import bit_block_scaled_nvfp4_amd as nv  # noqa: E402

nv.LIB_PATH = os.path.abspath(sys.argv[1])

import pytest  # noqa: E402

sys.exit(pytest.main([os.path.join(ROOT, "tests", "test_abi.py"), "-q", "-p", "no:cacheprovider",
                      *sys.argv[2:]]))
