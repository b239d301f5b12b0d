"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

capi.cpp (argument validation, workspace layout, kv_cache_bytes) is rebuilt with host-only
sanitizers and linked with the unchanged GPU objects into _build/libcsakv_hostsan.so; the
host-side test suite of the C ABI (tests/test_capi.py) then runs against it in a child
process with the sanitizer runtime preloaded.  Any sanitizer report aborts the child."""
import os
import subprocess
import sys

import pytest

from compressed_sparse_kv_csa_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _stale(target, sources):
    return not os.path.exists(target) or any(os.path.getmtime(s) > os.path.getmtime(target)
                                             for s in sources)


@pytest.fixture(scope="module")
def sanitized_library():
    srcs = [os.path.join(B.CSRC, f) for f in os.listdir(B.CSRC)] + [os.path.join(ROOT, "include", "csakv.h")]
    objs = [os.path.join(B.BUILD, os.path.basename(s) + ".o") for s in B._sources()]
    if any(_stale(o, srcs) for o in objs):
        B.build()
    if _stale(B.SAN_LIB, srcs + objs):
        B.build_host_sanitized()
    return B.SAN_LIB


def _run(lib, args):
    env = dict(os.environ)
    env.update(LD_PRELOAD=B.host_sanitizer_runtime(), CSAKV_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=600)


def test_the_sanitized_library_is_the_one_loaded(sanitized_library):
    r = _run(sanitized_library, ["-c", (
        "import compressed_sparse_kv_csa_amd as ck; ck.lib(); "
        "maps = open('/proc/self/maps').read(); "
        "print('hostsan' in maps, 'libclang_rt.asan' in maps)")])
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.split() == ["True", "True"], r.stdout


def test_capi_suite_under_host_sanitizers(sanitized_library):
    r = _run(sanitized_library, ["-m", "pytest", "tests/test_capi.py", "-q", "-p", "no:cacheprovider"])
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout
