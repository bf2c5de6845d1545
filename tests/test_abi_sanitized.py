"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds libmtfm_san.so (sanitizers on the host compilation only; the device
code is unchanged) and runs the argument-checking tests of test_abi.py against
it in a child process with the ASan runtime preloaded: every entry point's
validation, layout planning and error paths run instrumented, and any
out-of-bounds access, use after free or undefined behaviour aborts the child.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    libs = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return libs[-1] if libs else None


@pytest.mark.skipif(_asan_runtime() is None, reason="clang ASan runtime not installed")
def test_abi_checks_under_host_sanitizers():
    from hybrid_masked_attention_amd import build
    lib = build.build(jobs=8, sanitize=True)
    env = dict(os.environ, MTFM_LIB=lib, LD_PRELOAD=_asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # the child proves it runs the sanitized library with the runtime mapped
    probe = ("import sys; sys.path.insert(0, %r); from hybrid_masked_attention_amd import binding as B; "
             "B.lib(); maps = open('/proc/self/maps').read(); "
             "assert B.LIB_PATH.endswith('libmtfm_san.so') and 'libmtfm_san.so' in maps and 'asan' in maps; "
             "print('sanitized library loaded')" % ROOT)
    r = subprocess.run([sys.executable, "-c", probe], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
                        "-p", "no:cacheprovider"], env=env, capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
