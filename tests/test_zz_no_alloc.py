"""GPU checks of attn_paged_decode_noalloc, the paged decode whose split-KV
partials live in the library's per-GPU static scratch instead of a workspace
the caller allocates.

Its outputs must equal those of the workspace entry points (attn_paged_decode
and attn_paged_decode_gqa, which run the same kernels with the same split
count) bit for bit, on consecutive calls of decreasing size (the second call
finds the first one's partials in the scratch), and agree with the oracle to
the paged-decode tolerance. Calls after the first on a device must not change
the device's free memory.
"""

import ctypes
import math

import pytest
import torch

import oracle
from workloads import PagedSpec, paged_inputs

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
TOL_LSE = 1e-3


@pytest.fixture(scope="module")
def api():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import attention_tiled_qk_amd as m
    return m


def say(msg):
    print(msg, flush=True)


# A larger call (16 sequences x 8 heads, 4 queries each, lengths U[100, 3000],
# the library's split count: 16 splits, 4.2 MB of partials), then smaller ones.
BIG = PagedSpec("noalloc_big_16seq_8h_q4", 16, 8, 4, 128, 91, len_lo=100, len_hi=3000)
SMALL = PagedSpec("noalloc_small_3seq_4h_q1", 3, 4, 1, 128, 92, len_lo=17, len_hi=1000)
GQA = PagedSpec("noalloc_gqa_5seq_16qh_4kvh_q2", 5, 4, 2, 128, 93, len_lo=2, len_hi=2500,
                q_heads=16)


def _dev(inp):
    return [t.cuda() for t in (inp.q, inp.k_pool, inp.v_pool, inp.block_tables, inp.seq_lens)]


def _noalloc(api, d, splits, causal, scale, o, lse):
    """One call of attn_paged_decode_noalloc through the C ABI."""
    q, kp, vp, bt, sl = d
    B, Hq, q_len, D = q.shape
    nblk, Hkv = kp.shape[0], kp.shape[1]
    st = api.lib.attn_paged_decode_noalloc(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kp.data_ptr()),
        ctypes.c_void_p(vp.data_ptr()), ctypes.c_void_p(bt.data_ptr()),
        ctypes.c_void_p(sl.data_ptr()), ctypes.c_void_p(o.data_ptr()),
        ctypes.c_void_p(lse.data_ptr()), B, Hq, Hkv, q_len, D, nblk, bt.shape[1], 16,
        int(causal), float(scale), int(splits), api.ATTN_BF16,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, api.lib.attn_status_string(st).decode()


def _with_workspace(api, d, splits, causal, scale):
    q, kp, vp, bt, sl = d
    return api.attn_paged_decode(q, kp, vp, bt, sl, causal=causal, scale=scale,
                                 num_splits=splits, return_lse=True)


def _outputs(d):
    q = d[0]
    B, Hq, q_len, _ = q.shape
    return torch.empty_like(q), torch.empty(B, Hq, q_len, device=q.device, dtype=torch.float32)


def _scratch_bytes(api, d, splits):
    q, kp, _, bt, _ = d
    B, Hq, q_len, D = q.shape
    return api.attn_paged_gqa_workspace_bytes(B, Hq, kp.shape[1], q_len, D, bt.shape[1], splits)


def _vs_oracle(inp, o, lse, causal, scale):
    ref_o, ref_lse = oracle.paged_attention(inp.q, inp.k_pool, inp.v_pool, inp.block_tables,
                                            inp.seq_lens, scale, causal)
    e = float((o.double().cpu() - torch.from_numpy(ref_o)).abs().max())
    el = float((lse.double().cpu() - torch.from_numpy(ref_lse)).abs().max())
    return e, el


@pytest.mark.parametrize("causal", [True, False])
def test_noalloc_matches_workspace_decode_on_shrinking_calls(api, causal):
    say(f"noalloc: big then small, causal={causal}")
    big, small = paged_inputs(BIG), paged_inputs(SMALL)
    db, ds = _dev(big), _dev(small)
    scale = 1.0 / math.sqrt(128)
    assert 0 < _scratch_bytes(api, db, 0) <= api.ATTN_NOALLOC_SCRATCH_BYTES
    assert 0 < _scratch_bytes(api, ds, 3) < _scratch_bytes(api, db, 0)
    ob, lb = _outputs(db)
    os_, ls = _outputs(ds)
    # two calls in a row, the second smaller, before any reference is computed
    _noalloc(api, db, 0, causal, scale, ob, lb)
    _noalloc(api, ds, 3, causal, scale, os_, ls)
    torch.cuda.synchronize()
    rb, rlb = _with_workspace(api, db, 0, causal, scale)
    rs, rls = _with_workspace(api, ds, 3, causal, scale)
    torch.cuda.synchronize()
    assert torch.equal(ob, rb) and torch.equal(lb, rlb)
    assert torch.equal(os_, rs) and torch.equal(ls, rls)
    for inp, o, lse, name in ((big, ob, lb, "big"), (small, os_, ls, "small")):
        e, el = _vs_oracle(inp, o, lse, causal, scale)
        say(f"  {name}: max|dO|={e:.3e} max|dlse|={el:.3e} vs the oracle")
        assert e <= TOL_BF16 and el <= TOL_LSE


def test_noalloc_grouped_query_and_single_split(api):
    say("noalloc: grouped-query with splits, then one split (no scratch)")
    inp = paged_inputs(GQA)
    d = _dev(inp)
    scale = 0.07
    for splits in (5, 1):
        o, lse = _outputs(d)
        _noalloc(api, d, splits, True, scale, o, lse)
        ro, rl = _with_workspace(api, d, splits, True, scale)
        torch.cuda.synchronize()
        assert torch.equal(o, ro) and torch.equal(lse, rl), splits
    e, el = _vs_oracle(inp, o, lse, True, scale)
    assert e <= TOL_BF16 and el <= TOL_LSE


def test_noalloc_binding_and_free_memory(api):
    """Through the Python binding, with outputs given: repeated calls leave the
    device's free memory as it was after the first one."""
    say("noalloc: binding, free memory across calls")
    inp = paged_inputs(SMALL)
    q, kp, vp, bt, sl = _dev(inp)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], device=q.device, dtype=torch.float32)
    api.attn_paged_decode_noalloc(q, kp, vp, bt, sl, num_splits=4, o=o, lse=lse)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    alloc0 = torch.cuda.memory_allocated()
    for _ in range(3):
        api.attn_paged_decode_noalloc(q, kp, vp, bt, sl, num_splits=4, o=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0
    assert torch.cuda.memory_allocated() == alloc0
    ro, rl = api.attn_paged_decode(q, kp, vp, bt, sl, num_splits=4, return_lse=True)
    assert torch.equal(o, ro) and torch.equal(lse, rl)


def test_noalloc_refuses_partials_beyond_the_scratch(api):
    """Refused on the host with ATTN_ERR_SCRATCH; nothing is launched."""
    c = api.ATTN_NOALLOC_SCRATCH_BYTES
    B, H, q_len = 64, 40, 16
    q = torch.zeros(B, H, q_len, 128, device="cuda", dtype=torch.bfloat16)
    kp = torch.zeros(4, H, 16, 128, device="cuda", dtype=torch.bfloat16)
    bt = torch.zeros(B, 4096, device="cuda", dtype=torch.int32)
    sl = torch.full((B,), 16, device="cuda", dtype=torch.int32)
    assert api.attn_paged_gqa_workspace_bytes(B, H, H, q_len, 128, 4096, 64) > c
    with pytest.raises(api.AttnError) as ei:
        api.attn_paged_decode_noalloc(q, kp, kp, bt, sl, num_splits=64)
    assert ei.value.status == -10
