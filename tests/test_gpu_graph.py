"""The library under HIP graph capture.

The entry points allocate nothing and never synchronise, so a caller can
capture them: a paged decode with split-KV (the attention kernel plus the
merge kernel) and a prefill are captured once into a graph and replayed with new
inputs copied into the captured buffers; every replay must equal the eager
call on the same inputs bit for bit. Eager work runs between the replays.
A second graph holds a serving step with state: an FP8 append of one token
per sequence (which may re-encode a block's older slots when its scale
grows), an FP8 decode with splits over the cache it just wrote, and a ragged
chunked prefill; each replay starts from a snapshot of the cache, and the
outputs and the cache it leaves must equal those of eager calls from the same
snapshot.
"""

import math

import pytest
import torch

from workloads import PagedSpec, paged_inputs, paged_inputs_fp8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import attention_tiled_qk_amd as m
    return m


def test_paged_decode_and_prefill_replay_from_a_graph(api):
    spec = PagedSpec("graph", 4, 3, 2, 128, seed=123, len_lo=100, len_hi=900, num_splits=4)
    inp = paged_inputs(spec)
    dq, dk, dv, dt, dl = (t.cuda() for t in (inp.q, inp.k_pool, inp.v_pool, inp.block_tables,
                                              inp.seq_lens))
    B, H, ql, D = inp.q.shape
    ws = torch.empty(api.attn_paged_workspace_bytes(B, H, ql, D, dt.shape[1], 4) // 4,
                     device="cuda")
    o = torch.empty_like(dq)
    lse = torch.empty((B, H, ql), device="cuda")
    g = torch.Generator().manual_seed(5)
    pq, pk, pv = (torch.randn(2, 2, 300, 128, generator=g).to(torch.bfloat16).cuda()
                  for _ in range(3))
    po = torch.empty_like(pq)

    def step():
        api.attn_paged_decode(dq, dk, dv, dt, dl, num_splits=4, o=o, lse=lse, workspace=ws)
        api.attn_prefill(pq, pk, pv, causal=True, o=po)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for r in range(3):
        # new inputs into the captured buffers, eager work in between
        dq.copy_(torch.randn(dq.shape, generator=g).to(torch.bfloat16))
        pq.copy_(torch.randn(pq.shape, generator=g).to(torch.bfloat16))
        _ = (dk.float().sum() + 1).item()
        graph.replay()
        torch.cuda.synchronize()
        o_g, lse_g, po_g = o.clone(), lse.clone(), po.clone()
        step()  # eager on the same inputs
        torch.cuda.synchronize()
        assert torch.equal(o_g, o) and torch.equal(lse_g, lse), f"decode replay {r}"
        assert torch.equal(po_g, po), f"prefill replay {r}"
    # and the results are attention, not stale buffers
    assert torch.isfinite(o.float()).all() and math.isfinite(float(lse.min()))


def test_fp8_serving_step_replays_from_a_graph(api):
    spec = PagedSpec("graph_fp8", 3, 2, 1, 128, seed=321, len_lo=40, len_hi=400, num_splits=3)
    inp = paged_inputs_fp8(spec)
    q8, kc, vc, ks, vs, dt, dl = (t.cuda() for t in (inp.q, inp.k_codes, inp.v_codes,
                                                      inp.k_scale, inp.v_scale,
                                                      inp.block_tables, inp.seq_lens))
    B, H, _, D = inp.q.shape
    g = torch.Generator().manual_seed(17)
    kn = torch.randn(B, H, 1, D, generator=g).to(torch.bfloat16).cuda()
    vn = torch.randn(B, H, 1, D, generator=g).to(torch.bfloat16).cuda()
    ws8 = torch.empty(api.attn_paged_gqa_workspace_bytes(B, H, H, 1, D, dt.shape[1], 3) // 4,
                      device="cuda")
    o8 = torch.empty_like(q8)
    lse8 = torch.empty((B, H, 1), device="cuda")

    cspec = PagedSpec("graph_chunk", 3, 2, 1, 128, seed=322, len_lo=200, len_hi=600)
    cinp = paged_inputs(cspec)
    pk, pv, pt, pl = (t.cuda() for t in (cinp.k_pool, cinp.v_pool, cinp.block_tables,
                                         cinp.seq_lens))
    qlens = (50, 1, 120)
    cu = torch.tensor([0, 50, 51, 171], dtype=torch.int32, device="cuda")
    qv = torch.randn(sum(qlens), H, D, generator=g).to(torch.bfloat16).cuda()
    ov = torch.empty_like(qv)

    def step():
        api.attn_paged_append_fp8(kn, vn, kc, vc, ks, vs, dt, dl)
        api.attn_paged_decode_fp8(q8, kc, vc, ks, vs, dt, dl, num_splits=3, o=o8, lse=lse8,
                                  workspace=ws8)
        api.attn_paged_prefill_varlen(qv, pk, pv, pt, pl, cu, max(qlens), o=ov)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    cache = (kc, vc, ks, vs)
    for r in range(3):
        # a new token (larger values each time, so block scales grow) and new queries
        kn.copy_((torch.randn(kn.shape, generator=g) * (2.0 + r)).to(torch.bfloat16))
        vn.copy_((torch.randn(vn.shape, generator=g) * (2.0 + r)).to(torch.bfloat16))
        q8.copy_(torch.randn(q8.shape, generator=g).to(torch.bfloat16))
        qv.copy_(torch.randn(qv.shape, generator=g).to(torch.bfloat16))
        snap = [t.clone() for t in cache]
        _ = (pk.float().sum() + 1).item()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (o8, lse8, ov, *cache)]
        for t, c in zip(cache, snap):
            t.copy_(c)
        step()  # eager from the same cache
        torch.cuda.synchronize()
        for name, a, b in zip(("o", "lse", "chunk o", "k codes", "v codes", "k scales",
                               "v scales"), got, (o8, lse8, ov, *cache)):
            assert torch.equal(a, b), f"replay {r}: {name} differs from the eager call"
    assert torch.isfinite(o8.float()).all() and torch.isfinite(ov.float()).all()
