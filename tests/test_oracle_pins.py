"""Pins of the CPU oracle against facts the pages and the mathematics fix.

None of these re-runs the oracle's own formula: they use pure-Python scalar
loops written from the textbook definition, a library routine (torch's
scaled_dot_product_attention on float64), closed forms, invariants, and the
paging figure of the iopencloud.com page (section 3.2). ``test_oracle_mutants``
plants plausible mistakes in copies of the oracle and shows these pins catch
every one of them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import PagedSpec, paged_inputs, permute_pool

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- helpers ---

def brute_attention(q, k, v, scale, causal):
    """Textbook softmax attention with Python floats, no max subtraction.

    softmax(scale q k^T) v row by row ([P2] §一), with the bottom-right causal
    rule: query t of Lq sees key j of Lk iff j <= Lk - Lq + t.
    """
    lq, lk, dv = len(q), len(k), len(v[0])
    out, lses = [], []
    for t in range(lq):
        w = []
        for j in range(lk):
            if causal and j > lk - lq + t:
                w.append(None)
                continue
            s = 0.0
            for c in range(len(q[t])):
                s += q[t][c] * k[j][c]
            w.append(math.exp(scale * s))
        z = sum(x for x in w if x is not None)
        if z == 0.0:
            out.append([0.0] * dv)
            lses.append(-math.inf)
            continue
        row = [0.0] * dv
        for j, x in enumerate(w):
            if x is None:
                continue
            for c in range(dv):
                row[c] += (x / z) * v[j][c]
        out.append(row)
        lses.append(math.log(z))
    return np.array(out), np.array(lses)


def rnd(rng, *shape):
    return rng.standard_normal(shape)


# --------------------------------------------- checks usable on any attn ---
# Each takes ``attn(q, k, v, scale, causal) -> (o, lse)`` and raises on failure.

TINY_CASES = [(1, 1, 1, True), (3, 3, 2, True), (4, 7, 3, True), (5, 5, 4, False),
              (2, 8, 4, True), (8, 8, 4, True), (6, 3, 2, False)]


def check_brute(attn):
    rng = np.random.default_rng(7)
    for lq, lk, d, causal in TINY_CASES:
        q, k, v = rnd(rng, lq, d), rnd(rng, lk, d), rnd(rng, lk, d)
        scale = 0.7
        o, lse = attn(q, k, v, scale, causal)
        ob, lb = brute_attention(q.tolist(), k.tolist(), v.tolist(), scale, causal)
        np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
        fin = np.isfinite(lb)
        np.testing.assert_allclose(lse[fin], lb[fin], rtol=0, atol=1e-13)
        assert np.all(np.isneginf(lse[~fin]))


def check_sdpa(attn):
    rng = np.random.default_rng(11)
    for lq, lk, d, causal in [(37, 37, 16, True), (5, 40, 16, True), (33, 29, 8, False), (64, 64, 64, True)]:
        q, k, v = rnd(rng, lq, d), rnd(rng, lk, d), rnd(rng, lk, d)
        scale = 1.0 / math.sqrt(d)
        o, _ = attn(q, k, v, scale, causal)
        tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (q, k, v))
        mask = None
        if causal:
            t = torch.arange(lq)[:, None]
            j = torch.arange(lk)[None, :]
            mask = (j <= (lk - lq) + t)[None, None]
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
        np.testing.assert_allclose(o, ref[0, 0].numpy(), rtol=0, atol=1e-12)


def check_closed_forms(attn):
    rng = np.random.default_rng(3)
    lq, lk, d = 9, 13, 5
    q, k, v = rnd(rng, lq, d), rnd(rng, lk, d), rnd(rng, lk, d)
    # scale 0 and K == 0: every visible key has equal weight
    for qq, kk, sc in [(q, k, 0.0), (q, np.zeros_like(k), 0.9)]:
        o, lse = attn(qq, kk, v, sc, True)
        for t in range(lq):
            n = lk - lq + t + 1
            np.testing.assert_allclose(o[t], v[:n].mean(axis=0), rtol=0, atol=1e-13)
            assert abs(lse[t] - math.log(n)) < 1e-13
    # first causal row of a square problem sees only key 0
    o, _ = attn(rnd(rng, lk, d), k, v, 0.8, True)
    assert np.array_equal(o[0], v[0])
    # one query, one key: the output is that key's value, lse is its score
    o, lse = attn(q[:1], k[:1], v[:1], 0.5, False)
    assert np.array_equal(o[0], v[0])
    assert abs(lse[0] - 0.5 * float(q[0] @ k[0])) < 1e-13
    # one key dominates by delta: output within (n-1) e^-delta 2 max|V| of it
    delta = 30.0
    kd = np.zeros((lk, d))
    qd = np.zeros((1, d))
    qd[0, 0] = 1.0
    kd[4, 0] = delta
    o, _ = attn(qd, kd, v, 1.0, False)
    bound = (lk - 1) * math.exp(-delta) * 2 * np.abs(v).max()
    assert np.abs(o[0] - v[4]).max() <= bound


def check_causal_future_blind(attn):
    rng = np.random.default_rng(5)
    lq, lk, d = 6, 10, 4
    q, k, v = rnd(rng, lq, d), rnd(rng, lk, d), rnd(rng, lk, d)
    o, lse = attn(q, k, v, 0.6, True)
    for t in range(lq):
        lim = lk - lq + t
        if lim + 1 >= lk:
            continue
        k2, v2 = k.copy(), v.copy()
        k2[lim + 1:] += 100.0
        v2[lim + 1:] = -v2[lim + 1:] * 3.0
        o2, lse2 = attn(q, k2, v2, 0.6, True)
        assert np.array_equal(o2[t], o[t]) and lse2[t] == lse[t]
    # and the last row does see the last key
    v3 = v.copy()
    v3[-1] += 1.0
    o3, _ = attn(q, k, v3, 0.6, True)
    assert not np.array_equal(o3[-1], o[-1])


ALL_CHECKS = [check_brute, check_sdpa, check_closed_forms, check_causal_future_blind]


# ------------------------------------------------------------ the tests ---

def oracle_attn(q, k, v, scale, causal):
    return oracle.dense_attention(q, k, v, scale, causal)


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_dense_pins(check):
    check(oracle_attn)


def test_p_rows_are_distributions():
    rng = np.random.default_rng(17)
    for lq, lk, causal in [(12, 12, True), (4, 30, True), (7, 9, False)]:
        q, k, v = rnd(rng, lq, 8), rnd(rng, lk, 8), rnd(rng, lk, 8)
        _, _, p = oracle.dense_attention(q, k, v, 0.35, causal, return_p=True)
        assert np.all(p >= 0)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        if causal:
            vis = np.arange(lk)[None, :] <= (lk - lq) + np.arange(lq)[:, None]
            assert np.all(p[~vis] == 0.0)
            assert np.all(p[vis] > 0)


def test_fully_masked_rows():
    rng = np.random.default_rng(2)
    q, k, v = rnd(rng, 6, 4), rnd(rng, 3, 4), rnd(rng, 3, 4)
    o, lse = oracle.dense_attention(q, k, v, 1.0, True)  # rows 0..2 see nothing
    assert np.all(o[:3] == 0.0) and np.all(np.isneginf(lse[:3]))
    assert np.all(np.isfinite(lse[3:]))


@pytest.mark.parametrize("bm,bn", [(64, 64), (16, 16), (48, 80), (1, 10**6), (7, 3)])
@pytest.mark.parametrize("lq,lk,causal", [(200, 200, True), (131, 131, False), (5, 173, True), (40, 97, False)])
def test_tiled_online_softmax_equals_one_shot(bm, bn, lq, lk, causal):
    """[P1] §2.2: the tiled recurrence gives the global softmax result."""
    rng = np.random.default_rng(lq * 1000 + lk)
    q, k, v = rnd(rng, lq, 32), rnd(rng, lk, 32), rnd(rng, lk, 32)
    o1, l1 = oracle.dense_attention(q, k, v, 0.2, causal)
    o2, l2 = oracle.online_softmax_attention(q, k, v, 0.2, causal, bm, bn)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-12)


def test_state_combination_is_associative_and_exact():
    """Folding per-block states in any grouping or order gives the one-shot
    softmax over all keys: ((a b) c) == (a (b c)) == (c (a b)), and O / l,
    m + log l equal dense attention over the union of the blocks."""
    rng = np.random.default_rng(17)
    q, k, v = rnd(rng, 9, 8), rnd(rng, 30, 8), rnd(rng, 30, 8)
    vis = oracle.causal_visibility(9, 30)
    cut = [(0, 7), (7, 19), (19, 30)]
    a, b, c = (oracle.block_state(q, k[x:y], v[x:y], 0.7, vis[:, x:y]) for x, y in cut)
    left = oracle.combine_states(oracle.combine_states(a, b), c)
    right = oracle.combine_states(a, oracle.combine_states(b, c))
    swapped = oracle.combine_states(c, oracle.combine_states(b, a))
    o_ref, lse_ref = oracle.dense_attention(q, k, v, 0.7, True)
    for m, l, o in (left, right, swapped):
        np.testing.assert_allclose(o / l[:, None], o_ref, rtol=0, atol=1e-13)
        np.testing.assert_allclose(m + np.log(l), lse_ref, rtol=0, atol=1e-13)
    # the empty state is the identity; a block no row sees leaves a state unchanged
    empty = (np.full(9, -np.inf), np.zeros(9), np.zeros((9, 8)))
    for x, y in zip(oracle.combine_states(empty, a), a):
        np.testing.assert_array_equal(x, y)
    masked = oracle.block_state(q, k, v, 0.7, np.zeros((9, 30), dtype=bool))
    for x, y in zip(oracle.combine_states(a, masked), a):
        np.testing.assert_array_equal(x, y)


def test_online_softmax_pins():
    """The tiled recurrence also passes the definition pins on its own."""
    for bm, bn in [(2, 3), (1, 1), (4, 4)]:
        for check in ALL_CHECKS:
            check(lambda q, k, v, s, c: oracle.online_softmax_attention(q, k, v, s, c, bm, bn))


def test_prefill_batches_heads_independently():
    g = torch.Generator().manual_seed(0)
    q, k, v = (torch.randn(2, 3, 20, 8, generator=g) for _ in range(3))
    o, lse = oracle.prefill(q, k, v, 0.3, True)
    for b in range(2):
        for h in range(3):
            ob, lb = brute_attention(q[b, h].tolist(), k[b, h].tolist(), v[b, h].tolist(), 0.3, True)
            np.testing.assert_allclose(o[b, h], ob, rtol=0, atol=1e-13)
            np.testing.assert_allclose(lse[b, h], lb, rtol=0, atol=1e-13)


def test_bf16_inputs_upcast_exactly():
    x = torch.randn(4, 4).to(torch.bfloat16)
    o, _ = oracle.dense_attention(x, x, x, 0.0, False)
    ref = np.array([[float(x[j, c]) for c in range(4)] for j in range(4)]).mean(axis=0)
    np.testing.assert_allclose(o[0], ref, rtol=0, atol=1e-15)


# ------------------------------------------------------------- paging ---

def _fixture():
    with open(os.path.join(GOLDEN, "paging_example.json")) as f:
        return json.load(f)


def test_paging_figure_fixture():
    """Hand-checkable gather on the block pool drawn in [P1] §3.2."""
    check_paging_fixture(oracle.paged_gather)


def check_paging_fixture(gather):
    fx = _fixture()
    bs = fx["block_size"]
    labels = fx["pool_labels"]
    # the tables must name exactly the slots labelled with that request, in order
    for req, table in fx["tables"].items():
        assert [labels[i] for i in table] == [f"{req}{n + 1}" for n in range(len(table))]
    # a pool whose every element encodes (physical block, slot, head, d)
    H, D = 2, 3
    nblk = len(labels)
    pool = np.zeros((nblk, H, bs, D))
    for i in range(nblk):
        for h in range(H):
            for s in range(bs):
                for c in range(D):
                    pool[i, h, s, c] = 1000 * i + 10 * s + 0.1 * h + 0.01 * c
    lens = {"A": 70, "B": 20}
    width = 5
    tables = np.full((2, width), -1)
    tables[0, :5] = fx["tables"]["A"]
    tables[1, :2] = fx["tables"]["B"]
    got = gather(pool, tables, [lens["A"], lens["B"]], bs)
    for b, req in enumerate(["A", "B"]):
        assert got[b].shape == (H, lens[req], D)
        for t in range(lens[req]):
            phys = fx["tables"][req][t // bs]
            for h in range(H):
                assert np.array_equal(got[b][h, t], pool[phys, h, t % bs])
    # spot values written out by hand: A's token 37 is block 5 ("A3"), slot 5
    assert got[0][0, 37, 0] == 1000 * 5 + 10 * 5
    # B's token 17 is block 9 ("B2"), slot 1
    assert got[1][1, 17, 2] == 1000 * 9 + 10 * 1 + 0.1 + 0.02


def _small_paged(seed=0, q_len=1, lens=(1, 16, 17, 100, 257), H=3, D=16, extra=5, prefix=0):
    spec = PagedSpec("t", len(lens), H, q_len, D, seed, len_lo=1, len_hi=1, extra_blocks=extra,
                     shared_prefix_blocks=prefix)
    inp = paged_inputs(spec)
    # override lengths with the requested ones, re-deriving tables
    g = torch.Generator().manual_seed(seed + 100)
    nb = [-(-n // 16) for n in lens]
    own = [n - prefix for n in nb]
    total = prefix + sum(own) + extra
    perm = torch.randperm(total, generator=g)
    width = max(nb)
    tables = torch.full((len(lens), width), -1, dtype=torch.int32)
    pos = prefix
    for b in range(len(lens)):
        row = torch.cat([perm[:prefix], perm[pos:pos + own[b]]])
        pos += own[b]
        tables[b, :row.numel()] = row.to(torch.int32)
    k_pool = torch.randn(total, H, 16, D, generator=g).to(torch.bfloat16)
    v_pool = torch.randn(total, H, 16, D, generator=g).to(torch.bfloat16)
    q = torch.randn(len(lens), H, q_len, D, generator=g).to(torch.bfloat16)
    inp.q, inp.k_pool, inp.v_pool, inp.block_tables = q, k_pool, v_pool, tables
    inp.seq_lens = torch.tensor(lens, dtype=torch.int32)
    return inp


def test_gather_unpermute_equals_contiguous():
    check_gather_contiguous(oracle.paged_gather)


def check_gather_contiguous(gather):
    inp = _small_paged()
    got = gather(inp.k_pool, inp.block_tables, inp.seq_lens)
    # build the contiguous cache directly from the pool, block by block
    for b, n in enumerate(inp.seq_lens.tolist()):
        blocks = [inp.k_pool[int(inp.block_tables[b, i])] for i in range(-(-n // 16))]
        contig = torch.cat(blocks, dim=1)[:, :n]  # [H, n, D]
        assert torch.equal(got[b], contig)


def test_shared_prefix_rows_identical():
    inp = _small_paged(lens=(40, 64, 90), prefix=2)
    got = oracle.paged_gather(inp.v_pool, inp.block_tables, inp.seq_lens)
    for b in range(1, 3):
        assert torch.equal(got[b][:, :32], got[0][:, :32])


@pytest.mark.parametrize("q_len", [1, 5, 16])
def test_paged_invariant_under_block_permutation(q_len):
    inp = _small_paged(q_len=q_len, lens=(20, 33, 130, 257))
    o1, l1 = oracle.paged_attention(inp.q, inp.k_pool, inp.v_pool, inp.block_tables, inp.seq_lens, 0.25, True)
    perm = permute_pool(inp, 99)
    assert not torch.equal(perm.block_tables, inp.block_tables)
    o2, l2 = oracle.paged_attention(perm.q, perm.k_pool, perm.v_pool, perm.block_tables, perm.seq_lens, 0.25, True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_paged_full_query_equals_causal_prefill():
    """q_len == seq_len over a fresh paged sequence is causal prefill."""
    n = 75
    inp = _small_paged(q_len=n, lens=(n,), H=2, D=8, extra=3)
    o, lse = oracle.paged_attention(inp.q, inp.k_pool, inp.v_pool, inp.block_tables, inp.seq_lens, 0.4, True)
    kc = oracle.paged_gather(inp.k_pool, inp.block_tables, inp.seq_lens)[0]
    vc = oracle.paged_gather(inp.v_pool, inp.block_tables, inp.seq_lens)[0]
    for h in range(2):
        ob, lb = brute_attention(inp.q[0, h].double().tolist(), kc[h].double().tolist(),
                                 vc[h].double().tolist(), 0.4, True)
        np.testing.assert_allclose(o[0, h], ob, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[0, h], lb, rtol=0, atol=1e-12)


@pytest.mark.parametrize("group,q_len", [(2, 1), (4, 3), (8, 1)])
def test_paged_gqa_equals_mha_on_repeated_kv_heads(group, q_len):
    """Grouped-query attention is multi-head attention on a pool whose every KV
    head is repeated for the query heads of its group."""
    hkv = 2
    inp = _small_paged(q_len=q_len, lens=(3, 17, 64, 100), H=hkv, D=8)
    g = torch.Generator().manual_seed(7)
    q = torch.randn(inp.q.shape[0], hkv * group, q_len, 8, generator=g).to(torch.bfloat16)
    o, lse = oracle.paged_attention(q, inp.k_pool, inp.v_pool, inp.block_tables, inp.seq_lens,
                                    0.3, True)
    kr = inp.k_pool.repeat_interleave(group, dim=1)
    vr = inp.v_pool.repeat_interleave(group, dim=1)
    o2, l2 = oracle.paged_attention(q, kr, vr, inp.block_tables, inp.seq_lens, 0.3, True)
    assert np.array_equal(o, o2) and np.array_equal(lse, l2)
    # and one head against scalar loops: query head 2*group-1 reads KV head 1
    kc = oracle.paged_gather(inp.k_pool, inp.block_tables, inp.seq_lens)
    vc = oracle.paged_gather(inp.v_pool, inp.block_tables, inp.seq_lens)
    hq = 2 * group - 1
    ob, lb = brute_attention(q[2, hq].double().tolist(), kc[2][1].double().tolist(),
                             vc[2][1].double().tolist(), 0.3, True)
    np.testing.assert_allclose(o[2, hq], ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[2, hq], lb, rtol=0, atol=1e-12)


def test_paged_varlen_equal_lengths_is_paged_attention():
    """With every sequence bringing q_len tokens, the ragged form is
    paged_attention on the token-major repacking of q."""
    inp = _small_paged(q_len=4, lens=(5, 17, 64, 100), H=3, D=8)
    B, H, lq, D = inp.q.shape
    packed = inp.q.permute(0, 2, 1, 3).reshape(B * lq, H, D)
    cu = torch.arange(0, B * lq + 1, lq, dtype=torch.int32)
    o, lse = oracle.paged_attention_varlen(packed, cu, inp.k_pool, inp.v_pool, inp.block_tables,
                                           inp.seq_lens, 0.3, True)
    o2, l2 = oracle.paged_attention(inp.q, inp.k_pool, inp.v_pool, inp.block_tables,
                                    inp.seq_lens, 0.3, True)
    assert np.array_equal(o, o2.transpose(0, 2, 1, 3).reshape(B * lq, H, D))
    assert np.array_equal(lse, l2.transpose(0, 2, 1).reshape(B * lq, H))


def test_paged_varlen_ragged_against_scalar_loops():
    """Query counts 3, 0, 1, 9: each sequence's rows against brute force."""
    inp = _small_paged(q_len=1, lens=(20, 33, 7, 50), H=2, D=8)
    qlens = [3, 0, 1, 9]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(qlens)]), dtype=torch.int32)
    g = torch.Generator().manual_seed(3)
    q = torch.randn(int(cu[-1]), 2, 8, generator=g).to(torch.bfloat16)
    o, lse = oracle.paged_attention_varlen(q, cu, inp.k_pool, inp.v_pool, inp.block_tables,
                                           inp.seq_lens, 0.5, True)
    assert np.all(np.isfinite(o)) and o.shape == (13, 2, 8)
    kc = oracle.paged_gather(inp.k_pool, inp.block_tables, inp.seq_lens)
    vc = oracle.paged_gather(inp.v_pool, inp.block_tables, inp.seq_lens)
    for b in (0, 2, 3):
        a, e = int(cu[b]), int(cu[b + 1])
        for h in range(2):
            ob, lb = brute_attention(q[a:e, h].double().tolist(), kc[b][h].double().tolist(),
                                     vc[b][h].double().tolist(), 0.5, True)
            np.testing.assert_allclose(o[a:e, h], ob, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[a:e, h], lb, rtol=0, atol=1e-12)


def test_paged_varlen_gqa_equals_repeated_kv_heads():
    """Ragged grouped-query prefill is the ragged multi-head form on a pool
    whose every KV head is repeated for the query heads of its group."""
    inp = _small_paged(q_len=1, lens=(20, 33, 7, 50), H=2, D=8)
    group = 3
    qlens = [5, 0, 7, 12]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(qlens)]), dtype=torch.int32)
    g = torch.Generator().manual_seed(4)
    q = torch.randn(int(cu[-1]), 2 * group, 8, generator=g).to(torch.bfloat16)
    o, lse = oracle.paged_attention_varlen(q, cu, inp.k_pool, inp.v_pool, inp.block_tables,
                                           inp.seq_lens, 0.4, True)
    kr = inp.k_pool.repeat_interleave(group, dim=1)
    vr = inp.v_pool.repeat_interleave(group, dim=1)
    o2, l2 = oracle.paged_attention_varlen(q, cu, kr, vr, inp.block_tables, inp.seq_lens, 0.4,
                                           True)
    assert np.array_equal(o, o2) and np.array_equal(lse, l2)
    # query head 4 (group 1) of sequence 3 against scalar loops over KV head 1
    kc = oracle.paged_gather(inp.k_pool, inp.block_tables, inp.seq_lens)
    vc = oracle.paged_gather(inp.v_pool, inp.block_tables, inp.seq_lens)
    a, e = int(cu[3]), int(cu[4])
    ob, lb = brute_attention(q[a:e, 4].double().tolist(), kc[3][1].double().tolist(),
                             vc[3][1].double().tolist(), 0.4, True)
    np.testing.assert_allclose(o[a:e, 4], ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[a:e, 4], lb, rtol=0, atol=1e-12)


def test_paged_gqa_rejects_uneven_heads():
    inp = _small_paged(H=2, D=8)
    q = torch.zeros(inp.q.shape[0], 3, 1, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        oracle.paged_attention(q, inp.k_pool, inp.v_pool, inp.block_tables, inp.seq_lens, 0.3, True)


def test_paged_poison_never_read():
    spec = PagedSpec("p", 3, 2, 5, 16, 8, len_lo=5, len_hi=60, extra_blocks=4, poison=True)
    inp = paged_inputs(spec)
    assert torch.isnan(inp.k_pool.float()).any()
    o, lse = oracle.paged_attention(inp.q, inp.k_pool, inp.v_pool, inp.block_tables, inp.seq_lens, 0.25, True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


# ------------------------------------------------------ split and merge ---

def test_split_ranges_cover_once():
    for n in [1, 15, 16, 17, 100, 2048, 32768]:
        for s in [1, 2, 3, 16, 64]:
            r = oracle.split_ranges(n, s)
            assert len(r) == s
            covered = [t for a, b in r for t in range(a, b)]
            assert covered == list(range(n))
            assert all(a % 16 == 0 for a, b in r if b > a)
    # 2048 blocks into 16 splits: 128 blocks (2048 tokens) each
    assert oracle.split_ranges(32768, 16)[0] == (0, 2048)
    assert oracle.split_ranges(32768, 16)[15] == (30720, 32768)


@pytest.mark.parametrize("lq,lk,causal", [(1, 300, True), (5, 300, True), (5, 37, False), (16, 1000, True)])
def test_split_merge_equals_one_shot(lq, lk, causal):
    """FlashDecoding's split plus cross-split reduction gives the unsplit result."""
    check_split_merge(oracle.split_partials, oracle.lse_merge, lq, lk, causal)


def check_split_merge(split_partials, lse_merge, lq, lk, causal):
    rng = np.random.default_rng(lk + lq)
    q, k, v = rnd(rng, lq, 16), rnd(rng, lk, 16), rnd(rng, lk, 16)
    o1, l1 = oracle.dense_attention(q, k, v, 0.25, causal)
    nb = -(-lk // 16)
    for s in [1, 2, 3, 16, nb, nb + 3]:
        op, lp = split_partials(q, k, v, 0.25, causal, s)
        if s > nb:
            assert np.all(np.isneginf(lp[nb:])) and np.all(op[nb:] == 0)
        o2, l2 = lse_merge(op, lp)
        np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-12)


def test_merge_closed_forms():
    check_merge_closed_forms(oracle.lse_merge)


def check_merge_closed_forms(lse_merge):
    rng = np.random.default_rng(4)
    o_parts = rnd(rng, 4, 3, 8)
    # equal lse: plain mean of the partial outputs, lse + log S
    o, lse = lse_merge(o_parts, np.full((4, 3), 1.5))
    np.testing.assert_allclose(o, o_parts.mean(axis=0), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, 1.5 + math.log(4), rtol=0, atol=1e-14)
    # one live partial, the rest -inf: that partial comes back unchanged
    lp = np.full((4, 3), -np.inf)
    lp[2] = [0.3, -2.0, 7.0]
    o, lse = lse_merge(o_parts, lp)
    assert np.array_equal(o, o_parts[2]) and np.array_equal(lse, lp[2])
    # all -inf: zero output, -inf lse
    o, lse = lse_merge(o_parts, np.full((4, 3), -np.inf))
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    # two partials with lse differing by log 3: weights 3/4 and 1/4
    lp = np.zeros((2, 3))
    lp[0] = math.log(3.0)
    o, _ = lse_merge(o_parts[:2], lp)
    np.testing.assert_allclose(o, 0.75 * o_parts[0] + 0.25 * o_parts[1], rtol=0, atol=1e-14)
