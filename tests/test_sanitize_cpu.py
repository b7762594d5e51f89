"""CPU-only: the fp64 oracle and the host side of the C ABI, built with
AddressSanitizer and UndefinedBehaviorSanitizer (tests/sanitize/Makefile),
run their drivers cleanly: every entry point on seeded inputs and edge cases
(oracle), every host-side argument check (ABI), leak detection on."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("make") is None or not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs make and the ROCm compilers")
def test_sanitized_oracle_and_host_abi(tmp_path):
    r = subprocess.run(["make", "-s", "-C", os.path.join(ROOT, "tests", "sanitize"), "run", f"OUT={tmp_path}"],
                       capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "oracle sanitizer driver ok" in out and "abi sanitizer driver ok" in out, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
