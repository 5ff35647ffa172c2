"""The C-ABI checks of test_abi.py again, against the library built with host-side
AddressSanitizer (runtime.cpp's argument validation, workspace planning, tile choice and context
bookkeeping instrumented; device code untouched).  Runs in a child process that preloads the
compiler's ASan runtime; no GPU is needed or touched."""
import os
import subprocess
import sys

import pytest

from adaptive_looped_denoising_amd import build as hipbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

RUNNER = """
import sys
sys.path.insert(0, %r)
from adaptive_looped_denoising_amd import binding as B
B.load(%r)
import pytest
rc = pytest.main(["-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu", %r])
maps = open("/proc/self/maps").read()
# the instrumented library and the sanitizer runtime were the ones mapped, the plain library not
assert "libalodlm_asan.so" in maps and "libclang_rt.asan" in maps and "libalodlm.so" not in maps
sys.exit(rc)
"""


def test_abi_checks_under_host_address_sanitizer():
    rt = hipbuild.asan_runtime()
    if not rt or not os.path.exists(hipbuild.ASAN_LIB):
        pytest.skip("host-ASan library or ASan runtime not present (built by __graft_entry__.build())")
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt
    # Python itself keeps allocations alive until exit; report memory errors, not those leaks
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    code = RUNNER % (ROOT, hipbuild.ASAN_LIB, os.path.join(ROOT, "tests", "test_abi.py"))
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
