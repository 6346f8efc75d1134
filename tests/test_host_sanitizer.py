"""The C-ABI host layer under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): rpa_api.cpp is built by the host compiler with both sanitizers
and stand-in launchers (relative_bias_amd/build_hostsan.py), and the host ABI
tests (argument checks, planner, workspace sizes, the no-alloc entry's
refusals) are rerun against it in a Python process that preloads the
sanitizer runtimes.  Any sanitizer report fails the test."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_layer_is_clean_under_asan_and_ubsan():
    from relative_bias_amd import build_hostsan
    lib = build_hostsan.build()
    env = dict(os.environ)
    env.update(RPA_TEST_LIB=lib, LD_PRELOAD=":".join(build_hostsan.runtimes()),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    log = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, log
    assert "passed" in r.stdout, log
    for marker in ("AddressSanitizer", "runtime error:", "LeakSanitizer"):
        assert marker not in r.stdout + r.stderr, log
