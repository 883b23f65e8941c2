"""GPU parity of the paged-cache writes, and a cache driven end to end.

* attn_paged_append and attn_paged_copy_blocks are data movement: the pools
  they leave must equal the oracle's (paged_append, copy_blocks) bit for bit.
* A small serving loop: the host allocator hands out blocks, forks sequences
  (sharing a prefix), reports copy-on-write copies; the library copies blocks,
  appends chunks and single tokens, and runs chunked prefill and decode over
  the cache. Every attention output is compared with the oracle's dense
  attention over the sequence's own token history (max abs error 2e-2 for
  bf16 outputs, as in the other parity tests).
"""

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
BS = 16


@pytest.fixture(scope="module")
def api():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import attention_tiled_qk_amd as m
    return m


def say(msg):
    print(msg, flush=True)


def rand_bf16(g, *shape):
    return torch.randn(shape, generator=g, dtype=torch.float32).to(torch.bfloat16)


def layout(g, lens, nb_total, width):
    """Disjoint random block tables covering ``lens`` tokens, -1 padded."""
    perm = torch.randperm(nb_total, generator=g)
    tables = torch.full((len(lens), width), -1, dtype=torch.int32)
    pos = 0
    for b, n in enumerate(lens):
        m = -(-n // BS)
        tables[b, :m] = perm[pos:pos + m].to(torch.int32)
        pos += m
    assert pos <= nb_total
    return tables


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("n_new", [1, 5, 16, 37])
def test_append_bit_exact(api, D, n_new):
    g = torch.Generator().manual_seed(100 + n_new + D)
    H, width = 4, 8
    lens = [n_new, n_new + 3, 16 + n_new, 128, 97]
    lens = [min(n, width * BS) for n in lens]
    nb = 48
    say(f"append D={D} n_new={n_new} lens={lens}")
    tables = layout(g, lens, nb, width)
    k_pool, v_pool = rand_bf16(g, nb, H, BS, D), rand_bf16(g, nb, H, BS, D)
    k_new, v_new = rand_bf16(g, len(lens), H, n_new, D), rand_bf16(g, len(lens), H, n_new, D)
    sl = torch.tensor(lens, dtype=torch.int32)
    k_ref, v_ref = oracle.paged_append(k_pool, v_pool, tables, sl, k_new, v_new)
    kd, vd = k_pool.cuda(), v_pool.cuda()
    api.attn_paged_append(k_new.cuda(), v_new.cuda(), kd, vd, tables.cuda(), sl.cuda())
    torch.cuda.synchronize()
    assert torch.equal(kd.cpu(), k_ref) and torch.equal(vd.cpu(), v_ref)


def test_append_short_sequence_places_only_valid_positions(api):
    g = torch.Generator().manual_seed(7)
    H, D, nb, width = 2, 128, 8, 2
    tables = torch.tensor([[3, 5], [1, -1]], dtype=torch.int32)
    sl = torch.tensor([2, 20], dtype=torch.int32)  # sequence 0 is shorter than n_new = 6
    k_pool, v_pool = rand_bf16(g, nb, H, BS, D), rand_bf16(g, nb, H, BS, D)
    k_new, v_new = rand_bf16(g, 2, H, 6, D), rand_bf16(g, 2, H, 6, D)
    k_ref, v_ref = oracle.paged_append(k_pool, v_pool, tables, sl, k_new, v_new)
    kd, vd = k_pool.cuda(), v_pool.cuda()
    api.attn_paged_append(k_new.cuda(), v_new.cuda(), kd, vd, tables.cuda(), sl.cuda())
    torch.cuda.synchronize()
    assert torch.equal(kd.cpu(), k_ref) and torch.equal(vd.cpu(), v_ref)


@pytest.mark.parametrize("H,D", [(40, 128), (3, 64)])
def test_copy_blocks_bit_exact(api, H, D):
    g = torch.Generator().manual_seed(11)
    nb = 20
    k_pool, v_pool = rand_bf16(g, nb, H, BS, D), rand_bf16(g, nb, H, BS, D)
    src = torch.tensor([4, 9, 0, 17], dtype=torch.int32)
    dst = torch.tensor([1, 2, 19, 5], dtype=torch.int32)
    k_ref, v_ref = oracle.copy_blocks(k_pool, v_pool, src, dst)
    kd, vd = k_pool.cuda(), v_pool.cuda()
    api.attn_paged_copy_blocks(kd, vd, src.cuda(), dst.cuda())
    torch.cuda.synchronize()
    assert torch.equal(kd.cpu(), k_ref) and torch.equal(vd.cpu(), v_ref)


def _check_attention(o, lse, q, hist_k, hist_v, scale, seqs):
    """o [B, H, q_len, D] against dense attention over each history."""
    on = o.double().cpu().numpy()
    ln = lse.double().cpu().numpy()
    worst = 0.0
    for i, s in enumerate(seqs):
        k, v = hist_k[s], hist_v[s]
        for h in range(q.shape[1]):
            ro, rl = oracle.dense_attention(q[i, h], k[h], v[h], scale, True)
            worst = max(worst, float(np.abs(on[i, h] - ro).max()))
            assert np.abs(ln[i, h] - rl).max() < 1e-3
    assert worst <= TOL_BF16, worst
    return worst


def test_serving_loop_with_fork_and_copy_on_write(api):
    """Prefill in chunks, fork two sequences mid-block, decode with CoW."""
    g = torch.Generator().manual_seed(21)
    H, D, NB, S, W = 8, 128, 96, 6, 16
    scale = D ** -0.5
    alloc = api.KVCacheAllocator(NB, S, W)
    k_pool = torch.zeros((NB, H, BS, D), dtype=torch.bfloat16, device="cuda")
    v_pool = torch.zeros_like(k_pool)
    hist_k = {s: torch.zeros((H, 0, D), dtype=torch.bfloat16) for s in range(S)}
    hist_v = {s: torch.zeros((H, 0, D), dtype=torch.bfloat16) for s in range(S)}

    def grow(seqs, n):
        """Reserve n tokens for each of seqs, run their copies, append random K/V."""
        copies = []
        for s in seqs:
            copies += alloc.append(s, n)
        if copies:
            src = torch.tensor([a for a, _ in copies], dtype=torch.int32, device="cuda")
            dst = torch.tensor([b for _, b in copies], dtype=torch.int32, device="cuda")
            api.attn_paged_copy_blocks(k_pool, v_pool, src, dst)
        tables, lens = alloc.export()
        kn, vn = rand_bf16(g, len(seqs), H, n, D), rand_bf16(g, len(seqs), H, n, D)
        idx = torch.tensor(seqs)
        api.attn_paged_append(kn.cuda(), vn.cuda(), k_pool, v_pool, tables[idx].cuda(),
                              lens[idx].cuda())
        for i, s in enumerate(seqs):
            hist_k[s] = torch.cat([hist_k[s], kn[i]], dim=1)
            hist_v[s] = torch.cat([hist_v[s], vn[i]], dim=1)
        return tables[idx].cuda(), lens[idx].cuda(), len(copies)

    # chunked prefill of sequences 0..3: 3 chunks of 40 tokens each
    prompt = [0, 1, 2, 3]
    for c in range(3):
        tables, lens, _ = grow(prompt, 40)
        q = rand_bf16(g, len(prompt), H, 40, D)
        o, lse = api.attn_paged_prefill(q.cuda(), k_pool, v_pool, tables, lens, return_lse=True)
        torch.cuda.synchronize()
        on = o.double().cpu().numpy()
        for i, s in enumerate(prompt):
            for h in range(H):
                ro, _ = oracle.dense_attention(q[i, h], hist_k[s][h], hist_v[s][h], scale, True)
                assert np.abs(on[i, h] - ro).max() <= TOL_BF16
        say(f"prefill chunk {c} ok")
    # 120 tokens = 7.5 blocks: forks share a partly filled last block
    alloc.fork(0, 4)
    alloc.fork(1, 5)
    for s, p in ((4, 0), (5, 1)):
        hist_k[s], hist_v[s] = hist_k[p].clone(), hist_v[p].clone()
    n_copies = 0
    for step in range(20):
        seqs = list(range(S))
        tables, lens, nc = grow(seqs, 1)
        n_copies += nc
        q = rand_bf16(g, S, H, 1, D)
        o, lse = api.attn_paged_decode(q.cuda(), k_pool, v_pool, tables, lens, return_lse=True)
        torch.cuda.synchronize()
        _check_attention(o, lse, q, hist_k, hist_v, scale, seqs)
    # the first decode step copies the two shared partial blocks, and only then
    assert n_copies == 2
    say(f"decode ok, {n_copies} copy-on-write copies")
    # release a parent: the child keeps reading the shared prefix
    alloc.release(0)
    tables, lens, _ = grow([4], 1)
    q = rand_bf16(g, 1, H, 1, D)
    o, lse = api.attn_paged_decode(q.cuda(), k_pool, v_pool, tables, lens, return_lse=True)
    torch.cuda.synchronize()
    _check_attention(o, lse, q, hist_k, hist_v, scale, [4])


def test_append_full_chunk_shape(api):
    """The chunked-prefill shape (8 sequences x 40 heads, 512 new tokens after
    3584 cached): pools bit-exact with the oracle on sampled sequences."""
    g = torch.Generator().manual_seed(31)
    B, H, D, n_new, L = 8, 40, 128, 512, 4096
    width = L // BS
    nb = B * width
    tables = layout(g, [L] * B, nb, width)
    k_pool = torch.zeros((nb, H, BS, D), dtype=torch.bfloat16)
    v_pool = torch.zeros_like(k_pool)
    k_new, v_new = rand_bf16(g, B, H, n_new, D), rand_bf16(g, B, H, n_new, D)
    sl = torch.full((B,), L, dtype=torch.int32)
    kd, vd = k_pool.cuda(), v_pool.cuda()
    api.attn_paged_append(k_new.cuda(), v_new.cuda(), kd, vd, tables.cuda(), sl.cuda())
    torch.cuda.synchronize()
    for b in (0, 5):
        got_k = oracle.paged_gather(kd.cpu(), tables[b:b + 1], sl[b:b + 1])[0]
        got_v = oracle.paged_gather(vd.cpu(), tables[b:b + 1], sl[b:b + 1])[0]
        assert torch.equal(got_k[:, L - n_new:], k_new[b]) and torch.equal(got_v[:, L - n_new:], v_new[b])
        assert (got_k[:, :L - n_new] == 0).all()
