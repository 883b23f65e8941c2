"""CPU tests of the paged-cache writes and the host block allocator.

* The oracle's append / block copy are pinned by the [P1] §3.2 page-table
  figure (tests/golden/paging_example.json), by a round trip through the
  oracle's gather (itself pinned by that figure), and by splitting invariance.
* The allocator (attn_kv_cache_* in the C library; pure host code) is checked
  against the figure's tables, against hand-derived copy-on-write cases, and
  on random operation sequences against its invariants and a simulated cache
  whose contents are moved with the oracle's append and copy.
"""

import json
import os
import random

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
BS = 16


@pytest.fixture(scope="module")
def api():
    import attention_tiled_qk_amd as m
    return m


def token_rows(seq_id, start, n, H=2, D=4):
    """[H, n, D] rows whose values name (sequence, position, head, lane)."""
    out = np.zeros((H, n, D))
    for h in range(H):
        for t in range(n):
            out[h, t] = seq_id * 1e6 + (start + t) * 100 + h * 10 + np.arange(D)
    return out


# --------------------------------------------------------- oracle: append ---

def test_append_places_tokens_as_the_paging_figure_draws_them():
    with open(os.path.join(GOLDEN, "paging_example.json")) as f:
        fig = json.load(f)
    labels = fig["pool_labels"]
    tabs = fig["tables"]
    lens = {"A": 70, "B": 20}  # five and two blocks, the last ones partly filled
    H, D = 2, 4
    k = np.full((len(labels), H, BS, D), -1.0)
    v = np.full((len(labels), H, BS, D), -2.0)
    width = max(len(t) for t in tabs.values())
    table = np.full((2, width), -1)
    for i, r in enumerate("AB"):
        table[i, :len(tabs[r])] = tabs[r]
    # grow both requests in uneven chunks: 7, 30, then the rest
    done = {"A": 0, "B": 0}
    for chunk in (7, 30, 10 ** 6):
        new = {r: min(chunk, lens[r] - done[r]) for r in "AB"}
        n = max(new.values())
        if n == 0:
            break
        for i, r in enumerate("AB"):
            if new[r] == 0:
                continue
            kn = np.zeros((2, H, new[r], D))
            kn[i] = token_rows(i, done[r], new[r], H, D)
            sl = np.zeros(2, dtype=np.int64)
            sl[i] = done[r] + new[r]
            one = np.array([[-1] * width, [-1] * width])
            one[i] = table[i]
            k, v = oracle.paged_append(k, v, one, sl, kn, -kn)
            done[r] += new[r]
    for blk, lab in enumerate(labels):
        if lab is None:
            assert (k[blk] == -1).all() and (v[blk] == -2).all(), blk
            continue
        i = "AB".index(lab[0])
        logical = int(lab[1:]) - 1  # label A3 = third block of A
        for s in range(BS):
            p = logical * BS + s
            if p < lens[lab[0]]:
                want = token_rows(i, p, 1, H, D)[:, 0]
                assert np.array_equal(k[blk, :, s], want) and np.array_equal(v[blk, :, s], -want)
            else:
                assert (k[blk, :, s] == -1).all()


def test_append_then_gather_round_trip():
    rng = np.random.default_rng(0)
    H, D, nb = 3, 8, 40
    lens = np.array([1, 16, 17, 100])
    perm = rng.permutation(nb)
    table = np.full((4, 7), -1)
    pos = 0
    for b, n in enumerate(lens):
        m = -(-n // BS)
        table[b, :m] = perm[pos:pos + m]
        pos += m
    hist = [rng.standard_normal((H, n, D)) for n in lens]
    k = np.zeros((nb, H, BS, D))
    v = np.zeros((nb, H, BS, D))
    # prefill lens - 1 tokens padded to one n_new, then a one-token decode step
    n_new = int(lens.max()) - 1
    kn = np.zeros((4, H, n_new, D))
    for b, n in enumerate(lens):
        if n - 1 > 0:
            kn[b, :, n_new - (n - 1):] = hist[b][:, :n - 1]
    k, v = oracle.paged_append(k, v, table, lens - 1, kn, kn)
    step = np.stack([h[:, -1:] for h in hist])
    k, v = oracle.paged_append(k, v, table, lens, step, step)
    got = oracle.paged_gather(k, table, lens)
    for b in range(4):
        assert np.array_equal(got[b], hist[b])


def test_append_in_pieces_equals_append_at_once():
    rng = np.random.default_rng(1)
    H, D, nb = 2, 4, 12
    table = np.array([[3, 7, 1, 10], [0, 5, 2, -1]])
    lens = np.array([50, 33])
    n = 20
    kn = rng.standard_normal((2, H, n, D))
    vn = rng.standard_normal((2, H, n, D))
    k0 = rng.standard_normal((nb, H, BS, D))
    v0 = rng.standard_normal((nb, H, BS, D))
    k1, v1 = oracle.paged_append(k0, v0, table, lens, kn, vn)
    k2, v2 = k0, v0
    for a, b in ((0, 5), (5, 6), (6, 20)):
        k2, v2 = oracle.paged_append(k2, v2, table, lens - (n - b), kn[:, :, a:b], vn[:, :, a:b])
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2)


def test_append_skips_negative_positions():
    k = np.zeros((2, 1, BS, 1))
    kn = np.arange(1, 5, dtype=float).reshape(1, 1, 4, 1)
    k2, _ = oracle.paged_append(k, k, np.array([[1]]), np.array([2]), kn, kn)
    assert k2[1, 0, :2, 0].tolist() == [3.0, 4.0] and (k2[1, 0, 2:] == 0).all() and (k2[0] == 0).all()


def test_copy_blocks_preserves_what_a_rewritten_table_reads():
    rng = np.random.default_rng(2)
    k = rng.standard_normal((6, 2, BS, 4))
    v = rng.standard_normal((6, 2, BS, 4))
    k2, v2 = oracle.copy_blocks(k, v, [4, 1], [0, 5])
    table = np.array([[4, 1]])
    moved = np.array([[0, 5]])
    for a, b in ((k, k2), (v, v2)):
        assert np.array_equal(oracle.paged_gather(a, table, [32])[0],
                              oracle.paged_gather(b, moved, [32])[0])
        for blk in (1, 2, 3, 4):
            assert np.array_equal(a[blk], b[blk])


# ------------------------------------------------------------ allocator ---

def test_allocator_reproduces_the_paging_figure(api):
    """Interleaved growth and release give exactly the [P1] §3.2 tables."""
    with open(os.path.join(GOLDEN, "paging_example.json")) as f:
        fig = json.load(f)
    c = api.KVCacheAllocator(len(fig["pool_labels"]), 4, 8)
    A, B, C, D = 0, 1, 2, 3
    for seq, n in ((A, 32), (B, 16), (C, 32), (A, 16), (D, 16), (A, 32), (B, 16)):
        assert c.append(seq, n) == []
    c.release(C)
    c.release(D)
    tables, lens = c.export()
    assert tables[A, :5].tolist() == fig["tables"]["A"] and (tables[A, 5:] == -1).all()
    assert tables[B, :2].tolist() == fig["tables"]["B"] and (tables[B, 2:] == -1).all()
    assert lens.tolist() == [80, 32, 0, 0]
    empty = [i for i, lab in enumerate(fig["pool_labels"]) if lab is None]
    assert c.free_blocks() == len(empty)
    for i in range(len(fig["pool_labels"])):
        assert c.refs(i) == (0 if i in empty else 1)


def test_fork_shares_blocks_and_copies_the_partial_last_block(api):
    c = api.KVCacheAllocator(8, 3, 4)
    assert c.append(0, 20) == []            # blocks 0, 1 (block 1 holds 4 tokens)
    c.fork(0, 1)
    assert c.refs(0) == 2 and c.refs(1) == 2 and c.length(1) == 20
    assert c.append(1, 3) == [(1, 2)]        # child writes into shared block 1: copy to 2
    t, l = c.export()
    assert t[0, :2].tolist() == [0, 1] and t[1, :2].tolist() == [0, 2]
    assert (c.refs(0), c.refs(1), c.refs(2)) == (2, 1, 1)
    assert c.append(0, 1) == []              # parent now owns block 1 alone
    assert l.tolist()[:2] == [20, 23] and c.length(0) == 21
    c.release(0)
    assert (c.refs(0), c.refs(1)) == (1, 0) and c.free_blocks() == 8 - 2
    c.release(1)
    assert c.free_blocks() == 8


def test_fork_at_a_block_boundary_needs_no_copy(api):
    c = api.KVCacheAllocator(8, 2, 4)
    c.append(0, 32)
    c.fork(0, 1)
    assert c.append(1, 1) == [] and c.export()[0][1, :3].tolist() == [0, 1, 2]
    assert c.refs(0) == 2 and c.refs(2) == 1


def test_allocator_errors_leave_state_unchanged(api):
    AttnError = api.AttnError
    c = api.KVCacheAllocator(3, 2, 4)
    c.append(0, 40)                           # 3 blocks: pool exhausted
    before = c.export()
    with pytest.raises(AttnError) as e:
        c.append(1, 1)
    assert e.value.status == -9               # ATTN_ERR_NO_BLOCKS
    with pytest.raises(AttnError):
        c.append(0, 30)                       # past 4 blocks per sequence
    with pytest.raises(AttnError):
        c.append(2, 1)                        # no such sequence
    with pytest.raises(AttnError):
        c.fork(0, 0)
    c.fork(0, 1)
    with pytest.raises(AttnError):
        c.fork(0, 1)                          # child not empty
    with pytest.raises(AttnError) as e:
        c.append(1, 1)                        # copy-on-write needs a free block
    assert e.value.status == -9
    t, l = c.export()
    assert np.array_equal(t[0], before[0][0]) and np.array_equal(t[1], before[0][0])
    assert l.tolist() == [40, 40] and c.free_blocks() == 0
    with pytest.raises(ValueError):
        api.KVCacheAllocator(0, 1, 1)


def test_allocator_c_abi_argument_checks(api):
    import ctypes
    L = api.lib
    h = L.attn_kv_cache_create(4, 2, 2)
    try:
        n = ctypes.c_int(7)
        assert L.attn_kv_cache_append(h, 0, -1, None, None, 0, ctypes.byref(n)) == -2
        assert L.attn_kv_cache_append(h, 0, 1, None, None, 0, None) == -2
        assert L.attn_kv_cache_append(h, 0, 0, None, None, 0, ctypes.byref(n)) == 0 and n.value == 0
        assert L.attn_kv_cache_append(h, 0, 20, None, None, 0, ctypes.byref(n)) == 0
        assert L.attn_kv_cache_fork(h, 0, 1) == 0
        # a copy is needed but no room was given for it
        assert L.attn_kv_cache_append(h, 1, 1, None, None, 0, ctypes.byref(n)) == -6
        assert L.attn_kv_cache_length(h, 1) == 20
        assert L.attn_kv_cache_block_refs(h, 4) == -2
        assert L.attn_kv_cache_length(None, 0) == -2
        assert L.attn_kv_cache_free_blocks(None) == -1
        assert L.attn_kv_cache_export(h, None, None) == -1
    finally:
        L.attn_kv_cache_destroy(h)
    L.attn_kv_cache_destroy(None)


@pytest.mark.parametrize("seed", range(6))
def test_allocator_random_operations_keep_contents(api, seed):
    """Random append / fork / release with a simulated cache.

    Every append moves data the way a caller would: the reported copies with
    the oracle's copy_blocks, then the new tokens with the oracle's
    paged_append through the exported tables. After every step each sequence
    must read back exactly its own token history, and the reference counts
    must equal the number of tables holding each block.
    """
    rnd = random.Random(seed)
    NB, S, W, H, D = 24, 5, 6, 1, 2
    c = api.KVCacheAllocator(NB, S, W)
    k = np.full((NB, H, BS, D), np.nan)
    hist = [np.zeros((H, 0, D)) for _ in range(S)]
    uid = 0
    for _ in range(300):
        op = rnd.random()
        s = rnd.randrange(S)
        if op < 0.6:
            n = rnd.choice([1, 1, 1, 3, 16, 17, 40])
            try:
                copies = c.append(s, n)
            except api.AttnError as e:
                assert e.status in (-9, -2)
                continue
            if copies:
                k, _ = oracle.copy_blocks(k, k, [a for a, _ in copies], [b for _, b in copies])
            rows = np.zeros((H, n, D))
            for t in range(n):
                uid += 1
                rows[:, t] = uid
            tables, lens = (x.numpy() for x in c.export())
            kn = np.zeros((S, H, n, D))
            kn[s] = rows
            only = np.full_like(tables, -1)
            only[s] = tables[s]
            sl = np.zeros(S, dtype=np.int64)
            sl[s] = lens[s]
            k, _ = oracle.paged_append(k, k, only, sl, kn, kn)
            hist[s] = np.concatenate([hist[s], rows], axis=1)
        elif op < 0.75:
            empty = [i for i in range(S) if c.length(i) == 0 and i != s]
            if empty and c.length(s) > 0:
                d = rnd.choice(empty)
                c.fork(s, d)
                hist[d] = hist[s].copy()
        else:
            c.release(s)
            hist[s] = np.zeros((H, 0, D))
        tables, lens = (x.numpy() for x in c.export())
        used = {}
        for i in range(S):
            assert lens[i] == hist[i].shape[1]
            nblk = -(-int(lens[i]) // BS)
            assert (tables[i, :nblk] >= 0).all() and (tables[i, nblk:] == -1).all()
            assert len(set(tables[i, :nblk].tolist())) == nblk
            for bid in tables[i, :nblk].tolist():
                used[bid] = used.get(bid, 0) + 1
            got = oracle.paged_gather(k, tables[i:i + 1], lens[i:i + 1])[0]
            assert np.array_equal(got, hist[i])
        for bid in range(NB):
            assert c.refs(bid) == used.get(bid, 0)
        assert c.free_blocks() == NB - len(used)
