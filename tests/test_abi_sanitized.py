"""The C ABI's host side under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): tests/test_abi.py -- symbol exports, status strings, workspace
sizing and every argument-validation path -- run against the sanitizer build
of the library (libbasiskv_san.so: host code instrumented, -Werror), in a
separate Python process with the sanitizer runtime preloaded.  Any report
(heap or stack overflow, use after free, signed overflow, misaligned or null
access, ...) fails the test."""

import os
import subprocess
import sys

from sparse_decode_attention_latent_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_pass_under_asan_and_ubsan():
    if not os.path.exists(build.SAN_LIB):
        build.build_sanitized(verbose=False)
    runtime = build.asan_runtime()
    assert os.path.exists(runtime), runtime
    env = dict(os.environ, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from sparse_decode_attention_latent_amd import api\n"
            "api.LIB_PATH = %r\n"
            "import pytest\n"
            "sys.exit(pytest.main(['-q', '--noconftest', '-p', 'no:cacheprovider', %r]))\n"
            % (ROOT, build.SAN_LIB, os.path.join(ROOT, "tests", "test_abi.py")))
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in r.stdout
