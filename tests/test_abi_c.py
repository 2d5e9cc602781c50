"""The C ABI used from a plain C99 program (tests/native/abi_c.c): compiled
with gcc against include/pa.h, linked to libpa.so, run on the CPU."""

import ctypes
import os
import shutil
import subprocess

import pytest

from paged_kv_cache_462_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_program_uses_the_abi(tmp_path):
    lib = _lib.lib_path()
    assert os.path.exists(lib), "build the library first"
    exe = tmp_path / "abi_c"
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "native", "abi_c.c"), lib,
           f"-Wl,-rpath,{os.path.dirname(lib)}", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr + r.stdout
    assert "abi ok" in r.stdout
    # the ctypes binding lays the structs out as the C compiler does
    lay = {ln.split()[1]: [int(x) for x in ln.split()[2:]]
           for ln in r.stdout.splitlines() if ln.startswith("layout ")}
    T, L = _lib.PaTensor, _lib.PaLaunch
    assert lay["pa_tensor"] == [ctypes.sizeof(T), T.dtype.offset, T.ndim.offset, T.shape.offset,
                                T.stride.offset, T.scale.offset]
    assert lay["pa_launch"] == [ctypes.sizeof(L), L.workspace.offset, L.workspace_bytes.offset,
                                L.partition_tokens.offset, L.path.offset, L.error_flags.offset]
