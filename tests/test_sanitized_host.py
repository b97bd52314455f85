"""The host C++ (C ABI checks, block manager, planner, validation calls, step
preparation) under the address and undefined-behaviour sanitizers.

The pages' warning that a wrong reference count or block shows up as
corrupted attention rather than a crash (mercemay.com "Paged KV Cache
Allocation and the Block Table", "Sharing blocks between sequences") applies
to the host bookkeeping too: an out-of-bounds write in the block manager
would corrupt tables silently.  This test builds the host sources with g++
and -fsanitize=address,undefined (paged_kv_cache_115_amd/build.py,
build_host_sanitized; no kernels), then runs the CPU tests of the library
against that build in a child process with the sanitizer runtimes preloaded:
any heap or stack overflow, use after free or undefined behaviour aborts the
child and fails the test."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_TESTS = ["tests/test_host_library.py", "tests/test_boundary_checks.py", "tests/test_step_prepare.py",
              "tests/test_plan_advance.py", "tests/test_zz_no_alloc.py"]


def _runtime(name: str):
    gxx = shutil.which("g++")
    if gxx is None:
        return None
    path = subprocess.run([gxx, f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.timeout(900)
def test_host_library_under_asan_and_ubsan():
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("g++ or its sanitizer runtimes are not installed")
    sys.path.insert(0, os.path.join(ROOT, "paged_kv_cache_115_amd"))
    try:
        import build as pagedkv_build
    finally:
        sys.path.pop(0)
    lib = pagedkv_build.build_host_sanitized()
    env = dict(os.environ, LD_PRELOAD=f"{asan} {ubsan}", PAGEDKV_HOST_SANITIZED_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    # The child must really run the sanitized build with the runtimes loaded.
    probe = subprocess.run(
        [sys.executable, "-c",
         "import paged_kv_cache_115_amd as pk; m = open('/proc/self/maps').read(); "
         "assert 'libpagedkv_host_sanitized.so' in m and 'libpagedkv.so' not in m and 'libasan' in m, 'not sanitized'; "
         "print(pk.LIB_PATH)"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0, probe.stderr[-3000:]
    assert probe.stdout.strip() == lib
    res = subprocess.run([sys.executable, "-m", "pytest", *HOST_TESTS, "-x", "-q", "-m", "not gpu",
                          "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=800)
    out = res.stdout[-3000:] + res.stderr[-3000:]
    assert res.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out
