"""The library's C header and exports used from C, not through ctypes.

tests/c/abi_check.c is compiled with the host C compiler against
include/attn.h, linked with the built library, and run. It checks status
codes, host-side validation and the block allocator; nothing in it needs a GPU.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c_program_uses_the_abi(tmp_path):
    from attention_tiled_qk_amd import LIB_PATH
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    exe = tmp_path / "abi_check"
    libdir = os.path.dirname(LIB_PATH)
    cmd = [cc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_check.c"), "-o", str(exe),
           LIB_PATH, f"-Wl,-rpath,{libdir}"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert "abi_check ok" in r.stdout
