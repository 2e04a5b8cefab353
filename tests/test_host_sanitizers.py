"""The host-only tests -- C-ABI argument validation (test_abi_host.py) and bank-file I/O
(test_bank_io.py) -- rerun in a child process against the library built with
AddressSanitizer and UndefinedBehaviorSanitizer on its host code.  Any report fails the run:
UBSan findings are made fatal at compile time and ASan halts on the first error."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "latent_memory_long_amd"))
build_sanitized = pytest.importorskip("build_sanitized")


@pytest.mark.timeout(900)
def test_host_layer_under_asan_and_ubsan():
    lib = build_sanitized.build()
    env = dict(os.environ, MSA_LIBRARY=lib, LD_PRELOAD=build_sanitized.runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    probe = subprocess.run([sys.executable, "-c", "import ctypes, latent_memory_long_amd as m; "
                            "ctypes.CDLL(None).__asan_init; print(m.LIB_PATH)"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0, probe.stderr[-2000:]
    assert probe.stdout.strip().splitlines()[-1] == lib
    files = [os.path.join(ROOT, "tests", f) for f in ("test_abi_host.py", "test_bank_io.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                        *files], cwd=ROOT, env=env, capture_output=True, text=True, timeout=800)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
