"""The library under HIP graph capture.

The entry points allocate nothing and never synchronise, so a caller can
capture them: a paged decode with split-KV (the attention kernel plus the
merge kernel) and a prefill are captured once into a graph and replayed with new
inputs copied into the captured buffers; every replay must equal the eager
call on the same inputs bit for bit. Eager work runs between the replays.
"""

import math

import pytest
import torch

from workloads import PagedSpec, paged_inputs

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
