"""The C-ABI tests (tests/test_abi.py: argument checks, workspace layout,
error messages, struct layout; no kernel launch) against a build whose host
code carries AddressSanitizer (top_reduce_amd.build_asan), in a subprocess
with the sanitizer runtime preloaded. Passes when every ABI test passes and
the sanitizer reports nothing. CPU only."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_abi_under_host_address_sanitizer():
    from top_reduce_amd import build_asan
    lib = build_asan.build()
    env = dict(os.environ)
    env["LD_PRELOAD"] = build_asan.asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:detect_odr_violation=0:halt_on_error=1"
    env["TOP_REDUCE_LIB"] = lib
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                        "-q", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
