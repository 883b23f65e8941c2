"""Python face of the gfx950 tiled-attention library.

A thin ctypes binding over the C ABI in ``include/attn.h``: it checks tensor
placement and layout, allocates outputs with torch (device memory and streams
are all torch is used for), passes raw pointers and the current HIP stream,
and raises ``AttnError`` with the library's status text on failure. Every
step of the computation runs in the HIP kernels; there is no fallback path.
If the shared library has not been built, importing this package raises.
"""

import contextlib
import ctypes
import math
import os

import torch

from .build import LIB_PATH

__all__ = [
    "AttnError", "attn_prefill", "attn_paged_decode", "attn_paged_workspace_bytes",
    "attn_paged_decode_gqa", "attn_paged_gqa_workspace_bytes", "attn_paged_decode_noalloc",
    "ATTN_NOALLOC_SCRATCH_BYTES", "attn_paged_prefill",
    "attn_paged_prefill_varlen", "attn_paged_prefill_gqa",
    "attn_lse_merge", "attn_paged_gather", "attn_paged_append", "attn_paged_copy_blocks",
    "KVCacheAllocator", "attn_paged_append_fp8", "attn_paged_copy_blocks_fp8",
    "attn_paged_decode_fp8", "attn_paged_check_tables", "attn_paged_check_append",
    "attn_paged_check_ragged", "attn_paged_check_ids", "attn_version",
    "lib", "LIB_PATH",
    "ATTN_F32", "ATTN_BF16",
]

ATTN_F32 = 0
ATTN_BF16 = 1
# per-GPU scratch of attn_paged_decode_noalloc (ATTN_NOALLOC_SCRATCH_BYTES in attn.h)
ATTN_NOALLOC_SCRATCH_BYTES = 32 << 20

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it first (python attention_tiled_qk_amd/build.py "
        "or __graft_entry__.build()); there is no non-HIP implementation")

lib = ctypes.CDLL(LIB_PATH)

_p = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t

lib.attn_prefill.argtypes = [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _i, _p]
lib.attn_prefill.restype = _i
lib.attn_paged_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i]
lib.attn_paged_workspace_bytes.restype = _sz
lib.attn_paged_decode.argtypes = [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i,
                                  _f, _i, _p, _sz, _i, _p]
lib.attn_paged_decode.restype = _i
lib.attn_paged_gqa_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i, _i]
lib.attn_paged_gqa_workspace_bytes.restype = _sz
lib.attn_paged_decode_noalloc.argtypes = [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i,
                                          _i, _i, _f, _i, _i, _p]
lib.attn_paged_decode_noalloc.restype = _i
lib.attn_paged_decode_gqa.argtypes = [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i,
                                      _i, _f, _i, _p, _sz, _i, _p]
lib.attn_paged_decode_gqa.restype = _i
lib.attn_paged_prefill.argtypes = [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i,
                                   _f, _i, _p]
lib.attn_paged_prefill.restype = _i
lib.attn_paged_prefill_varlen.argtypes = [_p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i,
                                          _i, _i, _i, _f, _i, _p]
lib.attn_paged_prefill_varlen.restype = _i
lib.attn_paged_prefill_gqa.argtypes = [_p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i,
                                       _i, _i, _i, _f, _i, _p]
lib.attn_paged_prefill_gqa.restype = _i
lib.attn_lse_merge.argtypes = [_p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _p]
lib.attn_lse_merge.restype = _i
lib.attn_paged_gather.argtypes = [_p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _p]
lib.attn_paged_gather.restype = _i
lib.attn_paged_check_tables.argtypes = [_p, _p, _i, _i, _i, _i, _p, _p]
lib.attn_paged_check_tables.restype = _i
lib.attn_paged_check_append.argtypes = [_p, _p, _i, _i, _i, _i, _p, _p]
lib.attn_paged_check_append.restype = _i
lib.attn_paged_check_ragged.argtypes = [_p, _p, _i, _i, _i, _p, _p]
lib.attn_paged_check_ragged.restype = _i
lib.attn_paged_check_ids.argtypes = [_p, _p, _i, _i, _p, _p]
lib.attn_paged_check_ids.restype = _i
lib.attn_paged_append.argtypes = [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i, _p]
lib.attn_paged_append.restype = _i
lib.attn_paged_copy_blocks.argtypes = [_p, _p, _p, _p, _i, _i, _i, _i, _i, _p]
lib.attn_paged_copy_blocks.restype = _i
lib.attn_paged_append_fp8.argtypes = [_p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i,
                                      _p]
lib.attn_paged_append_fp8.restype = _i
lib.attn_paged_copy_blocks_fp8.argtypes = [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _p]
lib.attn_paged_copy_blocks_fp8.restype = _i
lib.attn_paged_decode_fp8.argtypes = [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i,
                                      _i, _i, _i, _f, _i, _p, _sz, _p]
lib.attn_paged_decode_fp8.restype = _i
lib.attn_kv_cache_create.argtypes = [_i, _i, _i]
lib.attn_kv_cache_create.restype = _p
lib.attn_kv_cache_destroy.argtypes = [_p]
lib.attn_kv_cache_destroy.restype = None
lib.attn_kv_cache_append.argtypes = [_p, _i, _i, _p, _p, _i, ctypes.POINTER(_i)]
lib.attn_kv_cache_append.restype = _i
lib.attn_kv_cache_fork.argtypes = [_p, _i, _i]
lib.attn_kv_cache_fork.restype = _i
lib.attn_kv_cache_release.argtypes = [_p, _i]
lib.attn_kv_cache_release.restype = _i
lib.attn_kv_cache_length.argtypes = [_p, _i]
lib.attn_kv_cache_length.restype = _i
lib.attn_kv_cache_free_blocks.argtypes = [_p]
lib.attn_kv_cache_free_blocks.restype = _i
lib.attn_kv_cache_block_refs.argtypes = [_p, _i]
lib.attn_kv_cache_block_refs.restype = _i
lib.attn_kv_cache_export.argtypes = [_p, _p, _p]
lib.attn_kv_cache_export.restype = _i
lib.attn_status_string.argtypes = [_i]
lib.attn_status_string.restype = ctypes.c_char_p
lib.attn_version.argtypes = []
lib.attn_version.restype = _i


class AttnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {lib.attn_status_string(status).decode()} (status {status})")


def attn_version():
    return lib.attn_version()


def _check(status, where):
    if status != 0:
        raise AttnError(status, where)


# Device type the tensors passed to the library must have. Only the binding's
# own CPU tests change it, to check argument validation without a GPU (with a
# stub in place of ``lib``, so nothing is launched).
_DEVICE_TYPE = "cuda"


def _dev(t, name, dtype=None, device=None, shape=None):
    """Check that t is a contiguous device tensor (of dtype, on device, of
    exactly shape, where given) and return it."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != _DEVICE_TYPE:
        raise ValueError(f"{name} must live on the GPU (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device} (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    return t


def _workspace(ws, need, device):
    """The split-KV scratch: allocated here when none is given and one is
    needed; a caller's tensor must be contiguous, on `device` and hold at
    least `need` bytes (any dtype). Returns (tensor or None, its bytes)."""
    if ws is None:
        if need <= 0:
            return None, 0
        ws = torch.empty(need // 4, device=device, dtype=torch.float32)
    _dev(ws, "workspace", device=device)
    nbytes = ws.numel() * ws.element_size()
    if nbytes < need:
        raise ValueError(f"workspace holds {nbytes} bytes, the call needs {need}")
    return ws, nbytes


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device, stream):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(dt):
    if dt == torch.float32:
        return ATTN_F32
    if dt == torch.bfloat16:
        return ATTN_BF16
    raise ValueError(f"unsupported dtype {dt}")


def attn_prefill(q, k, v, *, causal=True, scale=None, o=None, lse=None, return_lse=False,
                 stream=None):
    """Exact attention of q, k, v [B, H, L, D] (float32 or bfloat16).

    Returns o (and the float32 log-sum-exp [B, H, L] when ``return_lse``).
    """
    _dev(q, "q")
    if q.dim() != 4:
        raise ValueError("q, k, v must all be [B, H, L, D] of the same shape")
    _dev(k, "k", q.dtype, q.device, q.shape)
    _dev(v, "v", q.dtype, q.device, q.shape)
    B, H, L, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if o is None:
        o = torch.empty_like(q)
    _dev(o, "o", q.dtype, q.device, q.shape)
    if return_lse and lse is None:
        lse = torch.empty((B, H, L), device=q.device, dtype=torch.float32)
    if lse is not None:
        _dev(lse, "lse", torch.float32, q.device, (B, H, L))
    st = lib.attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, L, D,
                          int(bool(causal)), float(scale), _dtype_code(q.dtype),
                          _stream(q.device, stream))
    _check(st, "attn_prefill")
    return (o, lse) if (return_lse or lse is not None) else o


# With ATTN_CHECK_TABLES=1 in the environment, every paged call first counts
# on the device the table entries it would read out of range and raises
# instead of launching (a debugging mode: it waits for the count each call).
CHECK_TABLES = os.environ.get("ATTN_CHECK_TABLES", "0") == "1"


def _check_tables(block_tables, seq_lens, num_blocks, min_len, what, stream):
    if not CHECK_TABLES:
        return
    n_len, n_id = attn_paged_check_tables(block_tables, seq_lens, num_blocks, min_len=min_len,
                                          stream=stream)
    if n_len or n_id:
        raise ValueError(f"{what}: {n_len} sequence length(s) out of range and {n_id} block id(s) "
                         f"outside [0, {num_blocks}) in the tables (ATTN_CHECK_TABLES)")


def _check_append_tables(block_tables, seq_lens, num_blocks, n_new, what, stream):
    if not CHECK_TABLES:
        return
    n_len, n_id = attn_paged_check_append(block_tables, seq_lens, num_blocks, n_new, stream=stream)
    if n_len or n_id:
        raise ValueError(f"{what}: {n_len} sequence length(s) out of range and {n_id} written "
                         f"block id(s) neither -1 nor in [0, {num_blocks}) (ATTN_CHECK_TABLES)")


def _check_ragged(cu_q_lens, seq_lens, total_q, max_q_len, what, stream):
    if not CHECK_TABLES:
        return
    n_off, n_seq = attn_paged_check_ragged(cu_q_lens, seq_lens, total_q, max_q_len, stream=stream)
    if n_off or n_seq:
        raise ValueError(f"{what}: {n_off} query offset error(s) and {n_seq} sequence(s) with more "
                         f"queries than max_q_len or their length (ATTN_CHECK_TABLES)")


def _check_ids(src, dst, num_blocks, what, stream):
    if not CHECK_TABLES:
        return
    n_src, n_dst = attn_paged_check_ids(src, dst, num_blocks, stream=stream)
    if n_src or n_dst:
        raise ValueError(f"{what}: {n_src} src and {n_dst} dst block id(s) outside "
                         f"[0, {num_blocks}) (ATTN_CHECK_TABLES)")


def attn_paged_workspace_bytes(B, H, q_len, D, max_blocks_per_seq, num_splits=0):
    return int(lib.attn_paged_workspace_bytes(B, H, q_len, D, max_blocks_per_seq, num_splits))


def attn_paged_gqa_workspace_bytes(B, Hq, Hkv, q_len, D, max_blocks_per_seq, num_splits=0):
    return int(lib.attn_paged_gqa_workspace_bytes(B, Hq, Hkv, q_len, D, max_blocks_per_seq,
                                                  num_splits))


def _paged_decode_args(q, k_pool, v_pool, block_tables, seq_lens, scale, o, lse, return_lse):
    """Checks of the paged decode arguments; allocates o (and lse when asked
    for) if not given. Returns (B, Hq, Hkv, q_len, D, num_blocks, block_size,
    table width, scale, o, lse)."""
    _dev(q, "q", torch.bfloat16)
    dev = q.device
    _dev(k_pool, "k_pool", torch.bfloat16, dev)
    _dev(v_pool, "v_pool", torch.bfloat16, dev)
    _dev(block_tables, "block_tables", torch.int32, dev)
    _dev(seq_lens, "seq_lens", torch.int32, dev)
    if q.dim() != 4 or k_pool.dim() != 4 or v_pool.shape != k_pool.shape:
        raise ValueError("q must be [B, Hq, q_len, D] and the pools [num_blocks, Hkv, 16, D]")
    B, Hq, q_len, D = q.shape
    nblk, Hkv, bs, Dp = k_pool.shape
    if Dp != D or Hkv <= 0 or Hq % Hkv != 0:
        raise ValueError("pool head_dim must match q and pool heads must divide query heads")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or seq_lens.shape != (B,):
        raise ValueError("block_tables must be [B, W] and seq_lens [B]")
    width = block_tables.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if o is None:
        o = torch.empty_like(q)
    _dev(o, "o", torch.bfloat16, dev, q.shape)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq, q_len), device=dev, dtype=torch.float32)
    if lse is not None:
        _dev(lse, "lse", torch.float32, dev, (B, Hq, q_len))
    return B, Hq, Hkv, q_len, D, nblk, bs, width, scale, o, lse


def attn_paged_decode(q, k_pool, v_pool, block_tables, seq_lens, *, causal=True, scale=None,
                      num_splits=0, o=None, lse=None, return_lse=False, workspace=None,
                      stream=None):
    """Attention of q [B, H, q_len, D] (bf16) over a paged K/V cache.

    k_pool, v_pool [num_blocks, H, 16, D] bf16; block_tables [B, W] int32;
    seq_lens [B] int32 (key counts including the q_len new tokens). A float32
    workspace is allocated here when the split count needs one and none is given.
    When the pools hold fewer heads than q (a divisor of them), the call goes to
    attn_paged_decode_gqa (grouped-query attention).
    """
    B, Hq, Hkv, q_len, D, nblk, bs, width, scale, o, lse = _paged_decode_args(
        q, k_pool, v_pool, block_tables, seq_lens, scale, o, lse, return_lse)
    dev = q.device
    need = attn_paged_gqa_workspace_bytes(B, Hq, Hkv, q_len, D, width, num_splits)
    workspace, ws_bytes = _workspace(workspace, need, dev)
    common = (_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), _ptr(seq_lens), _ptr(o),
              _ptr(lse), B)
    tail = (q_len, D, nblk, width, bs, int(bool(causal)), float(scale), int(num_splits),
            _ptr(workspace), ws_bytes, ATTN_BF16, _stream(q.device, stream))
    _check_tables(block_tables, seq_lens, nblk, q_len, "attn_paged_decode", stream)
    if Hq == Hkv:
        st = lib.attn_paged_decode(*common, Hq, *tail)
        _check(st, "attn_paged_decode")
    else:
        st = lib.attn_paged_decode_gqa(*common, Hq, Hkv, *tail)
        _check(st, "attn_paged_decode_gqa")
    return (o, lse) if (return_lse or lse is not None) else o


def attn_paged_decode_noalloc(q, k_pool, v_pool, block_tables, seq_lens, *, causal=True,
                              scale=None, num_splits=0, o=None, lse=None, return_lse=False,
                              stream=None):
    """attn_paged_decode (multi-head or grouped-query) whose split-KV partials
    live in the library's per-GPU static scratch: the library call allocates
    no device memory. Pass o (and lse) to keep this wrapper from allocating
    them. Calls on one GPU that may overlap in time race on the scratch.
    Raises AttnError (ATTN_ERR_SCRATCH) when the partials exceed
    ATTN_NOALLOC_SCRATCH_BYTES."""
    B, Hq, Hkv, q_len, D, nblk, bs, width, scale, o, lse = _paged_decode_args(
        q, k_pool, v_pool, block_tables, seq_lens, scale, o, lse, return_lse)
    _check_tables(block_tables, seq_lens, nblk, q_len, "attn_paged_decode_noalloc", stream)
    # the first call on a GPU looks its scratch up with that GPU current
    ctx = torch.cuda.device(q.device) if q.device.type == "cuda" else contextlib.nullcontext()
    with ctx:
        st = lib.attn_paged_decode_noalloc(
            _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), _ptr(seq_lens), _ptr(o),
            _ptr(lse), B, Hq, Hkv, q_len, D, nblk, width, bs, int(bool(causal)), float(scale),
            int(num_splits), ATTN_BF16, _stream(q.device, stream))
    _check(st, "attn_paged_decode_noalloc")
    return (o, lse) if (return_lse or lse is not None) else o


def attn_paged_decode_gqa(q, k_pool, v_pool, block_tables, seq_lens, **kw):
    """attn_paged_decode with pools of fewer heads than q (grouped-query):
    q [B, Hq, q_len, D], pools [num_blocks, Hkv, 16, D] with Hkv dividing Hq."""
    if k_pool.dim() != 4 or q.dim() != 4 or k_pool.shape[1] >= q.shape[1]:
        raise ValueError("grouped-query decode needs pools with fewer heads than q")
    return attn_paged_decode(q, k_pool, v_pool, block_tables, seq_lens, **kw)


def attn_paged_prefill(q, k_pool, v_pool, block_tables, seq_lens, *, causal=True, scale=None,
                       o=None, lse=None, return_lse=False, stream=None):
    """Chunked prefill over a paged cache: q [B, H, q_len, D] (bf16), the
    q_len newest tokens of each sequence, attend its seq_lens[b] cached keys in
    k_pool, v_pool [num_blocks, H, 16, D] through block_tables [B, W] int32."""
    _dev(q, "q", torch.bfloat16)
    dev = q.device
    _dev(k_pool, "k_pool", torch.bfloat16, dev)
    _dev(v_pool, "v_pool", torch.bfloat16, dev)
    _dev(block_tables, "block_tables", torch.int32, dev)
    _dev(seq_lens, "seq_lens", torch.int32, dev)
    if q.dim() != 4 or k_pool.dim() != 4 or v_pool.shape != k_pool.shape:
        raise ValueError("q must be [B, H, q_len, D] and the pools [num_blocks, H, 16, D]")
    B, H, q_len, D = q.shape
    nblk, Hp, bs, Dp = k_pool.shape
    if Hp != H or Dp != D:
        raise ValueError("pool heads / head_dim must match q")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or seq_lens.shape != (B,):
        raise ValueError("block_tables must be [B, W] and seq_lens [B]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if o is None:
        o = torch.empty_like(q)
    _dev(o, "o", torch.bfloat16, dev, q.shape)
    if return_lse and lse is None:
        lse = torch.empty((B, H, q_len), device=dev, dtype=torch.float32)
    if lse is not None:
        _dev(lse, "lse", torch.float32, dev, (B, H, q_len))
    _check_tables(block_tables, seq_lens, nblk, q_len, "attn_paged_prefill", stream)
    st = lib.attn_paged_prefill(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
                                _ptr(seq_lens), _ptr(o), _ptr(lse), B, H, q_len, D, nblk,
                                block_tables.shape[1], bs, int(bool(causal)), float(scale),
                                ATTN_BF16, _stream(q.device, stream))
    _check(st, "attn_paged_prefill")
    return (o, lse) if (return_lse or lse is not None) else o


def attn_paged_prefill_varlen(q, k_pool, v_pool, block_tables, seq_lens, cu_q_lens, max_q_len, *,
                              causal=True, scale=None, o=None, lse=None, return_lse=False,
                              stream=None):
    """Ragged chunked prefill over a paged cache: q [total_q, H, D] (bf16,
    token-major), sequence b owning query tokens cu_q_lens[b] .. cu_q_lens[b+1]-1
    (int32 device, B + 1 entries); ``max_q_len`` is the largest of those counts.
    Returns o [total_q, H, D] (and lse [total_q, H] float32). When the pools hold
    fewer heads than q (a divisor of them), the call goes to
    attn_paged_prefill_gqa (grouped-query attention)."""
    _dev(q, "q", torch.bfloat16)
    dev = q.device
    _dev(k_pool, "k_pool", torch.bfloat16, dev)
    _dev(v_pool, "v_pool", torch.bfloat16, dev)
    _dev(block_tables, "block_tables", torch.int32, dev)
    _dev(seq_lens, "seq_lens", torch.int32, dev)
    _dev(cu_q_lens, "cu_q_lens", torch.int32, dev)
    if q.dim() != 3 or k_pool.dim() != 4 or v_pool.shape != k_pool.shape:
        raise ValueError("q must be [total_q, H, D] and the pools [num_blocks, H, 16, D]")
    total_q, H, D = q.shape
    nblk, Hp, bs, Dp = k_pool.shape
    if Dp != D or Hp <= 0 or H % Hp != 0:
        raise ValueError("pool head_dim must match q and pool heads must divide query heads")
    B = seq_lens.shape[0]
    if block_tables.dim() != 2 or block_tables.shape[0] != B or cu_q_lens.shape != (B + 1,):
        raise ValueError("block_tables must be [B, W], seq_lens [B] and cu_q_lens [B + 1]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if o is None:
        o = torch.empty_like(q)
    _dev(o, "o", torch.bfloat16, dev, q.shape)
    if return_lse and lse is None:
        lse = torch.empty((total_q, H), device=dev, dtype=torch.float32)
    if lse is not None:
        _dev(lse, "lse", torch.float32, dev, (total_q, H))
    head = (_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), _ptr(seq_lens),
            _ptr(cu_q_lens), _ptr(o), _ptr(lse), B, H)
    tail = (total_q, int(max_q_len), D, nblk, block_tables.shape[1], bs, int(bool(causal)),
            float(scale), ATTN_BF16, _stream(q.device, stream))
    _check_tables(block_tables, seq_lens, nblk, 0, "attn_paged_prefill_varlen", stream)
    _check_ragged(cu_q_lens, seq_lens, total_q, int(max_q_len), "attn_paged_prefill_varlen", stream)
    if Hp == H:
        _check(lib.attn_paged_prefill_varlen(*head, *tail), "attn_paged_prefill_varlen")
    else:
        _check(lib.attn_paged_prefill_gqa(*head, Hp, *tail), "attn_paged_prefill_gqa")
    return (o, lse) if (return_lse or lse is not None) else o


def attn_paged_prefill_gqa(q, k_pool, v_pool, block_tables, seq_lens, cu_q_lens, max_q_len, **kw):
    """attn_paged_prefill_varlen with pools of fewer heads than q (grouped-query):
    q [total_q, Hq, D], pools [num_blocks, Hkv, 16, D] with Hkv dividing Hq."""
    if k_pool.dim() != 4 or q.dim() != 3 or k_pool.shape[1] >= q.shape[1]:
        raise ValueError("grouped-query prefill needs pools with fewer heads than q")
    return attn_paged_prefill_varlen(q, k_pool, v_pool, block_tables, seq_lens, cu_q_lens,
                                     max_q_len, **kw)


def attn_lse_merge(o_part, lse_part, *, out_dtype=torch.bfloat16, o=None, lse=None,
                   return_lse=False, stream=None):
    """Merge o_part [B, H, q_len, S, D] / lse_part [B, H, q_len, S] (float32)."""
    _dev(o_part, "o_part", torch.float32)
    dev = o_part.device
    _dev(lse_part, "lse_part", torch.float32, dev)
    if o_part.dim() != 5 or lse_part.shape != o_part.shape[:4]:
        raise ValueError("o_part must be [B, H, q_len, S, D] and lse_part [B, H, q_len, S]")
    B, H, q_len, S, D = o_part.shape
    if o is None:
        o = torch.empty((B, H, q_len, D), device=dev, dtype=out_dtype)
    _dev(o, "o", None, dev, (B, H, q_len, D))
    if return_lse and lse is None:
        lse = torch.empty((B, H, q_len), device=dev, dtype=torch.float32)
    if lse is not None:
        _dev(lse, "lse", torch.float32, dev, (B, H, q_len))
    st = lib.attn_lse_merge(_ptr(o_part), _ptr(lse_part), _ptr(o), _ptr(lse), B, H, q_len, S, D,
                            _dtype_code(o.dtype), _stream(o_part.device, stream))
    _check(st, "attn_lse_merge")
    return (o, lse) if (return_lse or lse is not None) else o


def attn_paged_gather(pool, block_tables, seq_lens, max_seq_len, *, out=None, stream=None):
    """Copy each sequence's valid rows out of pool [N, H, 16, D] (bf16) into
    out [B, H, max_seq_len, D]; rows past seq_len are left as they were."""
    _dev(pool, "pool", torch.bfloat16)
    dev = pool.device
    _dev(block_tables, "block_tables", torch.int32, dev)
    _dev(seq_lens, "seq_lens", torch.int32, dev)
    if pool.dim() != 4 or block_tables.dim() != 2:
        raise ValueError("pool must be [N, H, 16, D] and block_tables [B, W]")
    nblk, H, bs, D = pool.shape
    B, width = block_tables.shape
    if seq_lens.shape != (B,):
        raise ValueError("seq_lens must be [B]")
    if out is None:
        out = torch.zeros((B, H, max_seq_len, D), device=dev, dtype=torch.bfloat16)
    _dev(out, "out", torch.bfloat16, dev, (B, H, max_seq_len, D))
    _check_tables(block_tables, seq_lens, nblk, 0, "attn_paged_gather", stream)
    st = lib.attn_paged_gather(_ptr(pool), _ptr(block_tables), _ptr(seq_lens), _ptr(out), B, H, D,
                               nblk, width, max_seq_len, _stream(pool.device, stream))
    _check(st, "attn_paged_gather")
    return out


def attn_paged_check_tables(block_tables, seq_lens, num_blocks, *, min_len=1, stream=None):
    """Count, on the device, what the paged calls would read out of range:
    returns (sequences whose length is below min_len or past the table's
    16 * width keys, table entries those calls read whose id lies outside
    [0, num_blocks)). Waits for the count (a debugging aid, not for hot loops)."""
    _dev(block_tables, "block_tables", torch.int32)
    _dev(seq_lens, "seq_lens", torch.int32, block_tables.device)
    if block_tables.dim() != 2 or seq_lens.shape != (block_tables.shape[0],):
        raise ValueError("block_tables must be [B, W] and seq_lens [B]")
    B, width = block_tables.shape
    bad = torch.empty(2, device=block_tables.device, dtype=torch.int32)
    st = lib.attn_paged_check_tables(_ptr(block_tables), _ptr(seq_lens), B, min_len, num_blocks, width,
                                     _ptr(bad), _stream(block_tables.device, stream))
    _check(st, "attn_paged_check_tables")
    n_len, n_id = bad.tolist()
    return n_len, n_id


def _counts(fn, args, device, where, stream):
    bad = torch.empty(2, device=device, dtype=torch.int32)
    _check(fn(*args, _ptr(bad), _stream(device, stream)), where)
    return tuple(bad.tolist())


def attn_paged_check_append(block_tables, seq_lens, num_blocks, n_new, *, stream=None):
    """Count, on the device, what an append of n_new tokens per sequence would
    write out of range: returns (lengths outside [0, 16 * width], entries the
    append writes through that are neither -1 nor in [0, num_blocks)). Waits
    for the count."""
    _dev(block_tables, "block_tables", torch.int32)
    _dev(seq_lens, "seq_lens", torch.int32, block_tables.device)
    if block_tables.dim() != 2 or seq_lens.shape != (block_tables.shape[0],):
        raise ValueError("block_tables must be [B, W] and seq_lens [B]")
    B, width = block_tables.shape
    return _counts(lib.attn_paged_check_append,
                   (_ptr(block_tables), _ptr(seq_lens), B, n_new, num_blocks, width),
                   block_tables.device, "attn_paged_check_append", stream)


def attn_paged_check_ragged(cu_q_lens, seq_lens, total_q, max_q_len, *, stream=None):
    """Count, on the device, the errors of a ragged call's packed query offsets:
    returns (offset errors -- cu[0] != 0, cu[B] != total_q, decreasing steps --,
    sequences with more queries than max_q_len or than their length). Waits for
    the count."""
    _dev(cu_q_lens, "cu_q_lens", torch.int32)
    _dev(seq_lens, "seq_lens", torch.int32, cu_q_lens.device)
    B = seq_lens.shape[0] if seq_lens.dim() == 1 else -1
    if B <= 0 or cu_q_lens.shape != (B + 1,):
        raise ValueError("seq_lens must be [B] and cu_q_lens [B + 1]")
    return _counts(lib.attn_paged_check_ragged,
                   (_ptr(cu_q_lens), _ptr(seq_lens), B, total_q, max_q_len),
                   cu_q_lens.device, "attn_paged_check_ragged", stream)


def attn_paged_check_ids(src, dst, num_blocks, *, stream=None):
    """Count, on the device, the ids of src and of dst outside [0, num_blocks).
    Waits for the count."""
    _dev(src, "src", torch.int32)
    _dev(dst, "dst", torch.int32, src.device)
    if src.dim() != 1 or dst.shape != src.shape:
        raise ValueError("src, dst must be 1-D of one length")
    return _counts(lib.attn_paged_check_ids, (_ptr(src), _ptr(dst), src.numel(), num_blocks),
                   src.device, "attn_paged_check_ids", stream)


def attn_paged_append(k_new, v_new, k_pool, v_pool, block_tables, seq_lens, *, stream=None):
    """Write k_new, v_new [B, H, n_new, D] (bf16) into the pools [N, H, 16, D]
    in place: token t of sequence b goes to position seq_lens[b] - n_new + t
    (seq_lens counts the new tokens) through block_tables [B, W] int32."""
    _dev(k_new, "k_new", torch.bfloat16)
    dev = k_new.device
    _dev(v_new, "v_new", torch.bfloat16, dev)
    _dev(k_pool, "k_pool", torch.bfloat16, dev)
    _dev(v_pool, "v_pool", torch.bfloat16, dev)
    _dev(block_tables, "block_tables", torch.int32, dev)
    _dev(seq_lens, "seq_lens", torch.int32, dev)
    if k_new.dim() != 4 or v_new.shape != k_new.shape or k_pool.dim() != 4 \
            or v_pool.shape != k_pool.shape:
        raise ValueError("k_new, v_new must be [B, H, n_new, D] and the pools [N, H, 16, D]")
    B, H, n_new, D = k_new.shape
    nblk, Hp, bs, Dp = k_pool.shape
    if Hp != H or Dp != D:
        raise ValueError("pool heads / head_dim must match the new tokens")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or seq_lens.shape != (B,):
        raise ValueError("block_tables must be [B, W] and seq_lens [B]")
    _check_append_tables(block_tables, seq_lens, nblk, n_new, "attn_paged_append", stream)
    st = lib.attn_paged_append(_ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool),
                               _ptr(block_tables), _ptr(seq_lens), B, H, n_new, D, nblk,
                               block_tables.shape[1], bs, ATTN_BF16,
                               _stream(k_new.device, stream))
    _check(st, "attn_paged_append")


def attn_paged_copy_blocks(k_pool, v_pool, src, dst, *, stream=None):
    """Copy physical block src[i] onto dst[i] in both pools (int32 device ids)."""
    _dev(k_pool, "k_pool", torch.bfloat16)
    dev = k_pool.device
    _dev(v_pool, "v_pool", torch.bfloat16, dev)
    _dev(src, "src", torch.int32, dev)
    _dev(dst, "dst", torch.int32, dev)
    if k_pool.dim() != 4 or v_pool.shape != k_pool.shape or src.dim() != 1 \
            or dst.shape != src.shape:
        raise ValueError("pools must be [N, H, 16, D] and src, dst 1-D of one length")
    nblk, H, _, D = k_pool.shape
    if src.numel() > 0:
        _check_ids(src, dst, nblk, "attn_paged_copy_blocks", stream)
    st = lib.attn_paged_copy_blocks(_ptr(k_pool), _ptr(v_pool), _ptr(src), _ptr(dst),
                                    src.numel(), nblk, H, D, ATTN_BF16,
                                    _stream(k_pool.device, stream))
    _check(st, "attn_paged_copy_blocks")


def _fp8_pools(k_pool, v_pool, k_scale, v_scale, device=None):
    _dev(k_pool, "k_pool", torch.uint8, device)
    device = k_pool.device
    _dev(v_pool, "v_pool", torch.uint8, device)
    _dev(k_scale, "k_scale", torch.float32, device)
    _dev(v_scale, "v_scale", torch.float32, device)
    if k_pool.dim() != 4 or v_pool.shape != k_pool.shape:
        raise ValueError("FP8 pools must be uint8 [num_blocks, H, 16, D]")
    if k_scale.shape != k_pool.shape[:2] or v_scale.shape != k_scale.shape:
        raise ValueError("scales must be float32 [num_blocks, H]")
    return k_pool.shape


def attn_paged_append_fp8(k_new, v_new, k_pool, v_pool, k_scale, v_scale, block_tables,
                          seq_lens, *, stream=None):
    """Quantise k_new, v_new [B, H, n_new, D] (bf16) into FP8 pools (uint8
    E4M3 codes [N, H, 16, D] with float32 scales [N, H]), in place."""
    _dev(k_new, "k_new", torch.bfloat16)
    dev = k_new.device
    _dev(v_new, "v_new", torch.bfloat16, dev)
    nblk, H, bs, D = _fp8_pools(k_pool, v_pool, k_scale, v_scale, dev)
    _dev(block_tables, "block_tables", torch.int32, dev)
    _dev(seq_lens, "seq_lens", torch.int32, dev)
    if k_new.dim() != 4 or v_new.shape != k_new.shape or k_new.shape[1] != H \
            or k_new.shape[3] != D:
        raise ValueError("k_new, v_new must be [B, H, n_new, D] matching the pools")
    B, _, n_new, _ = k_new.shape
    if block_tables.dim() != 2 or block_tables.shape[0] != B or seq_lens.shape != (B,):
        raise ValueError("block_tables must be [B, W] and seq_lens [B]")
    _check_append_tables(block_tables, seq_lens, nblk, n_new, "attn_paged_append_fp8", stream)
    st = lib.attn_paged_append_fp8(_ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool),
                                   _ptr(k_scale), _ptr(v_scale), _ptr(block_tables),
                                   _ptr(seq_lens), B, H, n_new, D, nblk, block_tables.shape[1],
                                   bs, _stream(k_new.device, stream))
    _check(st, "attn_paged_append_fp8")


def attn_paged_copy_blocks_fp8(k_pool, v_pool, k_scale, v_scale, src, dst, *, stream=None):
    """Copy FP8 block src[i] (codes and scales) onto dst[i] in both pools."""
    nblk, H, _, D = _fp8_pools(k_pool, v_pool, k_scale, v_scale)
    _dev(src, "src", torch.int32, k_pool.device)
    _dev(dst, "dst", torch.int32, k_pool.device)
    if src.dim() != 1 or dst.shape != src.shape:
        raise ValueError("src, dst must be 1-D of one length")
    if src.numel() > 0:
        _check_ids(src, dst, nblk, "attn_paged_copy_blocks_fp8", stream)
    st = lib.attn_paged_copy_blocks_fp8(_ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale),
                                        _ptr(src), _ptr(dst), src.numel(), nblk, H, D,
                                        _stream(k_pool.device, stream))
    _check(st, "attn_paged_copy_blocks_fp8")


def attn_paged_decode_fp8(q, k_pool, v_pool, k_scale, v_scale, block_tables, seq_lens, *,
                          causal=True, scale=None, num_splits=0, o=None, lse=None,
                          return_lse=False, workspace=None, stream=None):
    """Attention of q [B, Hq, q_len, D] (bf16) over FP8 pools (uint8 E4M3
    [N, Hkv, 16, D], float32 scales [N, Hkv]); Hkv divides Hq."""
    _dev(q, "q", torch.bfloat16)
    dev = q.device
    nblk, Hkv, bs, Dp = _fp8_pools(k_pool, v_pool, k_scale, v_scale, dev)
    _dev(block_tables, "block_tables", torch.int32, dev)
    _dev(seq_lens, "seq_lens", torch.int32, dev)
    if q.dim() != 4:
        raise ValueError("q must be [B, Hq, q_len, D]")
    B, Hq, q_len, D = q.shape
    if Dp != D or Hq % Hkv != 0:
        raise ValueError("pool head_dim must match q and pool heads must divide query heads")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or seq_lens.shape != (B,):
        raise ValueError("block_tables must be [B, W] and seq_lens [B]")
    width = block_tables.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if o is None:
        o = torch.empty_like(q)
    _dev(o, "o", torch.bfloat16, dev, q.shape)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq, q_len), device=dev, dtype=torch.float32)
    if lse is not None:
        _dev(lse, "lse", torch.float32, dev, (B, Hq, q_len))
    need = attn_paged_gqa_workspace_bytes(B, Hq, Hkv, q_len, D, width, num_splits)
    workspace, ws_bytes = _workspace(workspace, need, dev)
    _check_tables(block_tables, seq_lens, nblk, q_len, "attn_paged_decode_fp8", stream)
    st = lib.attn_paged_decode_fp8(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale),
                                   _ptr(v_scale), _ptr(block_tables), _ptr(seq_lens), _ptr(o),
                                   _ptr(lse), B, Hq, Hkv, q_len, D, nblk, width, bs,
                                   int(bool(causal)), float(scale), int(num_splits),
                                   _ptr(workspace), ws_bytes, _stream(q.device, stream))
    _check(st, "attn_paged_decode_fp8")
    return (o, lse) if (return_lse or lse is not None) else o


class KVCacheAllocator:
    """Host block allocator of a paged cache (the attn_kv_cache_* calls).

    Blocks are taken as sequences grow and returned on release; fork shares a
    sequence's blocks by reference count, and append reports the one block
    copy that copy-on-write needs as a (src, dst) pair.
    """

    def __init__(self, num_blocks, max_seqs, max_blocks_per_seq):
        self.num_blocks = num_blocks
        self.max_seqs = max_seqs
        self.max_blocks_per_seq = max_blocks_per_seq
        self._destroy = lib.attn_kv_cache_destroy  # kept for interpreter shutdown
        self._h = lib.attn_kv_cache_create(num_blocks, max_seqs, max_blocks_per_seq)
        if not self._h:
            raise ValueError("attn_kv_cache_create failed: sizes must be positive")

    def close(self):
        if getattr(self, "_h", None):
            self._destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def append(self, seq, n_tokens):
        """Reserve n_tokens more tokens for seq; returns the copies [(src, dst)]."""
        src = (ctypes.c_int32 * 1)()
        dst = (ctypes.c_int32 * 1)()
        n = _i(0)
        _check(lib.attn_kv_cache_append(self._h, seq, n_tokens, src, dst, 1, ctypes.byref(n)),
               "attn_kv_cache_append")
        return [(src[0], dst[0])] if n.value else []

    def fork(self, parent, child):
        _check(lib.attn_kv_cache_fork(self._h, parent, child), "attn_kv_cache_fork")

    def release(self, seq):
        _check(lib.attn_kv_cache_release(self._h, seq), "attn_kv_cache_release")

    def length(self, seq):
        r = lib.attn_kv_cache_length(self._h, seq)
        _check(min(r, 0), "attn_kv_cache_length")
        return r

    def free_blocks(self):
        return lib.attn_kv_cache_free_blocks(self._h)

    def refs(self, block):
        r = lib.attn_kv_cache_block_refs(self._h, block)
        _check(min(r, 0), "attn_kv_cache_block_refs")
        return r

    def export(self):
        """(block_tables [max_seqs, max_blocks_per_seq], seq_lens [max_seqs]) int32 CPU tensors."""
        tables = torch.empty((self.max_seqs, self.max_blocks_per_seq), dtype=torch.int32)
        lens = torch.empty((self.max_seqs,), dtype=torch.int32)
        _check(lib.attn_kv_cache_export(self._h, _ptr(tables), _ptr(lens)), "attn_kv_cache_export")
        return tables, lens
