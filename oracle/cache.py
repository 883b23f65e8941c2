"""Plain definitions of the paged-cache writes: appending tokens, copying blocks.

TEST INFRASTRUCTURE ONLY (see the package docstring). These are data
movement, not arithmetic: the results hold the input values bit for bit.

Readings taken where the pages leave a step open:
  * ``seq_lens`` passed to an append already counts the new tokens, so new
    token t of a sequence with n_new new tokens has absolute position
    seq_len - n_new + t -- the same convention the attention calls use for the
    position of query t.
  * a token whose position would be negative (seq_len < n_new) is not placed.
"""

import numpy as np

try:
    import torch
except ImportError:  # pragma: no cover
    torch = None


def _i64(x):
    if torch is not None and isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.int64).numpy()
    return np.asarray(x, dtype=np.int64)


def paged_append(k_pool, v_pool, block_tables, seq_lens, k_new, v_new, block_size=16):
    """Return copies of the pools with the new tokens written in.

    PagedAttention's cache ([P1] §3.2, [P3] Continuous Batching +
    PagedAttention item): token at position p of sequence b is stored in its
    logical block p // block_size, i.e. physical block block_tables[b][p //
    block_size], slot p % block_size. Writing the new tokens is that mapping
    applied to each of them in turn; nothing else in the pools changes.

    k_pool, v_pool [num_blocks, H, block_size, D]; k_new, v_new [B, H, n_new, D]
    (torch tensors or arrays, any dtype, copied unchanged).
    """
    tables = _i64(block_tables)
    lens = _i64(seq_lens)
    k_out = k_pool.clone() if hasattr(k_pool, "clone") else np.array(k_pool, copy=True)
    v_out = v_pool.clone() if hasattr(v_pool, "clone") else np.array(v_pool, copy=True)
    n_new = k_new.shape[2]
    for b in range(tables.shape[0]):
        for t in range(n_new):
            p = int(lens[b]) - n_new + t
            if p < 0:
                continue
            phys = int(tables[b][p // block_size])
            if phys < 0:
                continue
            k_out[phys, :, p % block_size, :] = k_new[b, :, t, :]
            v_out[phys, :, p % block_size, :] = v_new[b, :, t, :]
    return k_out, v_out


def copy_blocks(k_pool, v_pool, src, dst):
    """Return copies of the pools where block dst[i] holds block src[i]'s contents.

    The copy a sequence makes of a block it shares before writing into it
    ([P4], the subsection on paged memory management: reference-counted
    blocks, copy-on-write). Sources are read from the pools as they were
    before any copy of the call.
    """
    src = _i64(src)
    dst = _i64(dst)
    k_out = k_pool.clone() if hasattr(k_pool, "clone") else np.array(k_pool, copy=True)
    v_out = v_pool.clone() if hasattr(v_pool, "clone") else np.array(v_pool, copy=True)
    for s, d in zip(src, dst):
        k_out[int(d)] = k_pool[int(s)]
        v_out[int(d)] = v_pool[int(s)]
    return k_out, v_out
