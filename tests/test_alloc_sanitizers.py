"""The host block allocator and block manager under ThreadSanitizer and
AddressSanitizer + UndefinedBehaviorSanitizer (CPU).

tests/native/alloc_stress.cpp drives one allocator, one block manager and
one prefix cache from several threads (sequences with shared prefix
blocks, appends with copy-on-write, forks, frees, direct allocate / incref /
decref, exports; prefix matches, inserts, releases and evictions) and
checks the pool is whole at the end.  It is built here with g++ from
the allocator's source alone (host code, no device code involved)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "paged_kv_cache_462_amd", "csrc", "pa_alloc.cpp"),
       os.path.join(ROOT, "paged_kv_cache_462_amd", "csrc", "pa_prefix.cpp"),
       os.path.join(ROOT, "tests", "native", "alloc_stress.cpp")]

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")


@pytest.mark.parametrize("flags", [["-fsanitize=thread"], ["-fsanitize=address,undefined",
                                                           "-fno-sanitize-recover=all"]])
def test_allocator_under_sanitizer(tmp_path, flags):
    exe = tmp_path / "alloc_stress"
    cmd = ["g++", "-std=c++17", "-O1", "-g", *flags, "-I", os.path.join(ROOT, "include"),
           *SRC, "-o", str(exe), "-pthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1", ASAN_OPTIONS="detect_leaks=1")
    r = subprocess.run([str(exe), "8", "3000"], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ThreadSanitizer" not in r.stderr and "AddressSanitizer" not in r.stderr
    assert "runtime error" not in r.stderr
    assert "alloc stress ok" in r.stdout
