"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The library's host code -- argument validation and launch sizing
(csrc/attn_api.hip) and the block allocator (csrc/kv_cache.hip) -- is
compiled with ``-fsanitize=address,undefined`` for the host pass only (the
device code is built as usual), linked into a separate library, and driven by
three C programs built with the same sanitizers: the ABI walk-through
(tests/c/abi_check.c), a random allocator workload with invariant checks
(tests/c/alloc_fuzz.c) and every entry point under extreme sizes
(tests/c/validation_edges.c). A sanitizer report ends a program with a
non-zero status. The programs never launch on a GPU: the suite skips this
test where one is present, since calls that pass validation reach a launch.
"""

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_tiled_qk_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
SANITIZED = {"attn_api.hip", "kv_cache.hip", "table_check.hip"}
PROGRAMS = ["abi_check.c", "alloc_fuzz.c", "validation_edges.c"]


def _gpu_present():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.skipif(_gpu_present(), reason="calls that pass validation would launch on the GPU")
def test_host_code_under_sanitizers(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    clang = "/opt/rocm/llvm/bin/clang"
    if not os.path.exists(hipcc) or not os.path.exists(clang):
        pytest.skip("ROCm toolchain not found")
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_attn_build", os.path.join(ROOT, "attention_tiled_qk_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)

    def compile_one(src):
        obj = str(tmp_path / (src + ".o"))
        extra = HOST_SAN + ["-g"] if src in SANITIZED else []
        cmd = [hipcc, *b.FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        return obj

    with ThreadPoolExecutor(4) as ex:
        objs = list(ex.map(compile_one, b.SOURCES))
    lib = str(tmp_path / "libattn_san.so")
    r = subprocess.run([hipcc, f"--offload-arch={b.ARCH}", "-shared", "-fPIC", *objs, "-o", lib],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    for prog in PROGRAMS:
        exe = str(tmp_path / prog[:-2])
        cmd = [clang, "-std=c99", "-g", "-Wall", "-Werror", "-fsanitize=address,undefined",
               "-fno-sanitize-recover=all", "-I", INCLUDE, os.path.join(ROOT, "tests", "c", prog),
               "-o", exe, lib, f"-Wl,-rpath,{tmp_path}"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
        assert r.returncode == 0, f"{prog}:\n{r.stdout}\n{r.stderr[-4000:]}"
        assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr
        print(r.stdout.strip())
