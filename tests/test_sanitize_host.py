"""liblora's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): tests/sanitize/build_and_run.sh builds the library with both
sanitizers on its host code, links the C driver tests/sanitize/abi_driver.cpp
(every entry point's validation paths and the workspace planners over a grid
of shapes up to the size limits) and runs it."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SCRIPT = os.path.join(HERE, "sanitize", "build_and_run.sh")


@pytest.mark.skipif(not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")),
                    reason="hipcc not available")
def test_host_code_under_asan_and_ubsan(tmp_path):
    r = subprocess.run(["bash", SCRIPT, str(tmp_path)], capture_output=True, text=True,
                       timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "0 failures" in r.stdout, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
