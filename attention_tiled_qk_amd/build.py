"""Compile the HIP sources into the in-tree shared library (gfx950 only)."""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB_NAME = "libattn_tiled_qk.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU forms are kept out of the generated code. hipcc forwards
    # -Xclang to the host pass too (-Xarch_device refuses options that take an
    # argument), where LLVM prints that it ignores the unknown feature.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Werror", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]
SOURCES = [
    "attn_api.hip", "prefill_bf16.hip", "prefill_f32.hip", "paged.hip", "kv_append.hip",
    "kv_cache.hip", "table_check.hip",
]


def _hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build")
    return exe


def _compile(src, src_dir=CSRC, build_dir=BUILD_DIR):
    obj = os.path.join(build_dir, os.path.splitext(os.path.basename(src))[0] + ".o")
    cmd = [_hipcc(), *FLAGS, "-c", os.path.join(src_dir, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def link(objs, lib_path):
    """Link objects into the shared library lib_path (replaced atomically)."""
    tmp = lib_path + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib_path)
    return lib_path


def build(verbose=True):
    """Compile every kernel source and link libattn_tiled_qk.so next to this file."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    link(objs, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}", file=sys.stderr)
    return LIB_PATH


if __name__ == "__main__":
    build()
