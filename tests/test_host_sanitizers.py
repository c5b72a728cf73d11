"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

csa2_api.hip's argument checks are built with g++ into a host-check library whose kernel
launchers are stubs that refuse every launch; the ABI tests (tests/test_abi_cpu.py) then run
against it in a child process with the sanitizer runtimes preloaded, and any sanitizer
report fails the test. A call that passes every check reaches a stub and must come back as
a HIP error, which shows the stub library (not the kernels) was loaded."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="g++ is not installed")

PROBE = r"""
import ctypes, os
from compressed_kv_cache_csa2_amd import csa2 as C
assert C._LIB_PATH == os.environ["CSA2_LIBRARY"], C._LIB_PATH
F = 0x10000
st = C.lib.csa2_index_score(0, 1, 32, 128, F, F, F, 10, F, F, None, 0, 8, F, 16, None, 0, None, None)
msg = C.lib.csa2_last_error()
assert st != 0 and b"launch failed" in msg, (st, msg)
print("stub reached:", msg.decode())
"""


@pytest.fixture(scope="module")
def hostcheck(tmp_path_factory):
    sys.path.insert(0, ROOT)
    from compressed_kv_cache_csa2_amd import build
    lib = str(tmp_path_factory.mktemp("hostcheck") / "libcsa2_hostcheck.so")
    build.build_hostcheck(lib)
    env = dict(os.environ)
    env["CSA2_LIBRARY"] = lib
    env["LD_PRELOAD"] = " ".join(build.sanitizer_runtimes())
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    return lib, env


def _clean(out):
    for marker in ("AddressSanitizer", "runtime error:", "UndefinedBehaviorSanitizer"):
        assert marker not in out, out[-4000:]


def test_abi_tests_pass_under_asan_and_ubsan(hostcheck):
    lib, env = hostcheck
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_cpu.py"),
                        "-q", "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    _clean(out)


def test_valid_call_reaches_the_launch_stub(hostcheck):
    lib, env = hostcheck
    r = subprocess.run([sys.executable, "-c", PROBE], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "stub reached" in out
    _clean(out)
