"""The ABI tests again, against the host-sanitized build of the library
(AddressSanitizer and UBSan on the host code, -Xarch_host): every argument
check, byte-count and overlap computation of the validation path runs under
the sanitizers, on the CPU.  The sanitized library is built if missing or
older than the sources, and the tests run in a child process that preloads
the sanitizer runtime."""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from global_hybrid_causal_amd import build as B  # noqa: E402


def _stale() -> bool:
    if not os.path.exists(B.SAN_LIB):
        return True
    t = os.path.getmtime(B.SAN_LIB)
    sources = glob.glob(os.path.join(B.CSRC, "*")) + [os.path.join(ROOT, "include", "olmo3_attn.h")]
    return any(os.path.getmtime(p) > t for p in sources)


def test_abi_suite_under_host_sanitizers():
    try:
        runtime = B.sanitizer_runtime()
    except RuntimeError as e:  # no HIP toolchain
        pytest.skip(str(e))
    if runtime is None:
        pytest.skip("clang AddressSanitizer runtime not found")
    if _stale():
        B.build_host_sanitized()
    env = dict(os.environ, LD_PRELOAD=runtime, OLMO3_ATTN_LIB=B.SAN_LIB,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    # the child maps the sanitizer runtime and the sanitized library
    probe = ("from global_hybrid_causal_amd import attn as A; A.lib(); "
             "m = open('/proc/self/maps').read(); "
             "print('asan' if 'libclang_rt.asan' in m else 'no asan', "
             "'san-lib' if A.LIB_PATH in m else 'other lib')")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.split() == ["asan", "san-lib"], r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "failed" not in r.stdout, tail
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
