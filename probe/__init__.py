"""Read-bandwidth probe of the benchmark (not part of the attention library).

``probe_block_read`` reads listed blocks of a device buffer and nothing else,
so its rate is the ceiling that HBM sustains for the scattered 2-4 KiB block
reads of the paged kernels -- the bandwidth their roofline is measured
against ([P4], roofline and MBU). The kernel lives in ``block_read.hip`` and
is built into ``libattn_probe.so`` next to this file by ``build()``;
``bench.py`` and its GPU test load it from there.
"""

import ctypes
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn_probe.so")

_lib = None


def build(verbose=True):
    """Compile block_read.hip for gfx950 (the attention library's flags) and
    link libattn_probe.so."""
    root = os.path.dirname(HERE)
    if root not in sys.path:
        sys.path.insert(0, root)
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_attn_build", os.path.join(root, "attention_tiled_qk_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    bdir = os.path.join(b.BUILD_DIR, "probe")
    os.makedirs(bdir, exist_ok=True)
    obj = b._compile("block_read.hip", HERE, bdir)
    b.link([obj], LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}", file=sys.stderr)
    return LIB_PATH


def lib():
    """The loaded probe library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run probe.build() (or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        p, i = ctypes.c_void_p, ctypes.c_int
        L.probe_block_read.argtypes = [p, i, i, p, i, p, i, i, p]
        L.probe_block_read.restype = i
        _lib = L
    return _lib


def probe_block_read(buf, block_bytes, order, n_waves, *, nontemporal=False, sink=None,
                     stream=None):
    """Read the blocks of buf (uint8 device tensor, a whole number of
    block_bytes blocks) listed in order (int32 device tensor) with the default
    or the nontemporal cache policy. Returns sink [n_waves * 64] int32 whose
    XOR over all words is the XOR of every 32-bit word read."""
    import torch
    for t, name, dt in ((buf, "buf", torch.uint8), (order, "order", torch.int32)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or not t.is_contiguous() \
                or t.dtype != dt:
            raise ValueError(f"{name} must be a contiguous {dt} GPU tensor")
    if order.device != buf.device:
        raise ValueError("order must be on buf's device")
    if buf.numel() % block_bytes != 0:
        raise ValueError("buf must hold a whole number of blocks")
    if sink is None:
        sink = torch.empty(n_waves * 64, device=buf.device, dtype=torch.int32)
    if sink.device != buf.device or sink.dtype != torch.int32 or not sink.is_contiguous() \
            or sink.numel() < n_waves * 64:
        raise ValueError("sink must be a contiguous int32 tensor of n_waves * 64 words on buf's device")
    s = stream if stream is not None else torch.cuda.current_stream(buf.device)
    st = lib().probe_block_read(ctypes.c_void_p(buf.data_ptr()), buf.numel() // block_bytes,
                                block_bytes, ctypes.c_void_p(order.data_ptr()), order.numel(),
                                ctypes.c_void_p(sink.data_ptr()), n_waves, int(bool(nontemporal)),
                                ctypes.c_void_p(s.cuda_stream))
    if st != 0:
        raise RuntimeError(f"probe_block_read failed with status {st}")
    return sink
