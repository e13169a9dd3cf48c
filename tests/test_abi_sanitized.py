"""The C ABI's host-side argument handling under AddressSanitizer and
UndefinedBehaviorSanitizer: a sanitized build of the library (host code
instrumented, device code as usual) runs the CPU checks of test_abi_host.py in
a child process with the sanitizer runtime preloaded; any report aborts it."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_host_checks_under_sanitizers():
    from block_diffusion_drafter_target_amd import build
    lib = build.build_sanitized(verbose=False)
    env = dict(os.environ, DFLASH_LIB=lib, LD_PRELOAD=build.sanitizer_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       env=env, capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "passed" in r.stdout
