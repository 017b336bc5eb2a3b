"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer: the oracle pins and the
C ABI's CPU checks, each run against a build with the sanitizers on (tests/sanitize_host.py).
CPU only; skipped where a GPU is visible (the ABI checks pass fake device pointers)."""
import os
import sys

import pytest

pytestmark = pytest.mark.skipif(
    __import__("torch").cuda.device_count() > 0,
    reason="host-only check: the ABI checks pass fake device pointers")


def test_host_code_under_sanitizers(tmp_path):
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import sanitize_host
    assert sanitize_host.main(["--out", str(tmp_path)]) == 0
