"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): the library's argument validation, layout and planning code
(every host-side path tests/test_abi_cpu.py drives) is built with
-fsanitize=address,undefined for the host (device code as usual) and the ABI
tests run against it in a child process with the sanitizer runtime preloaded;
any report aborts that process."""
import glob
import os
import subprocess
import sys

from sparse_loop_attention_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _sanitized_library() -> str:
    out = build.SANITIZED_OUT
    srcs = glob.glob(os.path.join(build.CSRC, "*")) + [os.path.join(build.INCLUDE, "flashloop.h")]
    if not os.path.exists(out) or os.path.getmtime(out) < max(os.path.getmtime(f) for f in srcs):
        build.build(sanitize=True)
    return out


def test_abi_tests_pass_under_asan_and_ubsan():
    lib = _sanitized_library()
    env = dict(os.environ, LD_PRELOAD=build.sanitizer_runtime(), FLASHLOOP_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_cpu.py"), "-q", "-x",
                        "-p", "no:cacheprovider"], env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
