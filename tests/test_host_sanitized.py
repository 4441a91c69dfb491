"""The host bookkeeping under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): the library's host translation units (pool, plan, prefix cache,
C ABI layer) are built with both sanitizers, and the differential fuzzers of
the pool against the oracle -- [KVPool] append_or_allocate, copy_on_write,
release_sequence and the [PagedPool] validate invariants after every
operation, the window / rollback fuzz, the prefix-cache trace and the
decode work-list checks -- run against that build in a child process.  Any sanitizer report aborts the
child and fails the test.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FUZZERS = ["tests/test_abi_host.py", "tests/test_abi_window.py", "tests/test_abi_prefix.py", "tests/test_plan_host.py"]


def test_fuzzers_under_address_and_undefined_sanitizers():
    from paged_kv_cache_block_amd import sanitize_build
    try:
        runtime = sanitize_build.runtime_library()
    except FileNotFoundError as e:
        pytest.skip(str(e))
    lib = sanitize_build.build_sanitized()
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": runtime,
        "PA_TEST_SANITIZED_LIBRARY": lib,
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    probe = ("import conftest; conftest.pytest_configure(type('C', (), {'addinivalue_line': "
             "staticmethod(lambda *a: None)})()); from paged_kv_cache_block_amd import abi; abi.load(); "
             "maps = open('/proc/self/maps').read(); "
             "print('sanitized' if 'libpagedattn_sanitized.so' in maps and 'libclang_rt.asan' in maps else maps)")
    res = subprocess.run([sys.executable, "-c", probe], cwd=os.path.join(ROOT, "tests"), env=env,
                         capture_output=True, text=True, timeout=120)
    assert res.stdout.strip() == "sanitized", res.stdout[-2000:] + res.stderr[-2000:]
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider", *FUZZERS]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    report = res.stdout[-4000:] + res.stderr[-4000:]
    assert res.returncode == 0, report
    assert "ERROR: AddressSanitizer" not in report and "runtime error" not in report, report
    assert " passed" in res.stdout, report
