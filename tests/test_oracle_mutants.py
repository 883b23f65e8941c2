"""The oracle's pins are sharp enough to catch plausible mistakes.

Each mutant below is a copy of one oracle function with one planted mistake
(a dropped term, a wrong sign or index, a transposed operand, a misplaced
step). Every mutant must fail at least one of the pin checks that the real
oracle passes. Mistakes are planted here, on the CPU, in copies; the oracle
itself is untouched.
"""

import numpy as np
import pytest

import oracle
from tests.test_oracle_pins import (
    ALL_CHECKS,
    check_gather_contiguous,
    check_merge_closed_forms,
    check_paging_fixture,
    check_split_merge,
)


def _attn_variant(q, k, v, scale, causal, bug):
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    lq, lk = q.shape[0], k.shape[0]
    s = (q @ k.T) if bug == "no_scale" else scale * (q @ k.T)
    t = np.arange(lq)[:, None]
    j = np.arange(lk)[None, :]
    if bug == "strict_causal":
        vis = j < (lk - lq) + t
    elif bug == "top_left_causal":
        vis = j <= t
    elif bug == "off_by_one_causal":
        vis = j <= (lk - lq) + t + 1
    else:
        vis = j <= (lk - lq) + t
    if not causal:
        vis = np.ones((lq, lk), dtype=bool)
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1)
    empty = ~np.isfinite(m)
    ms = np.where(empty, 0.0, m)
    if bug == "exp_sign":
        p = np.where(vis, np.exp(ms[:, None] - s), 0.0)
    else:
        p = np.where(vis, np.exp(s - ms[:, None]), 0.0)
    l = p.sum(axis=1)
    ls = np.where(empty, 1.0, l)
    if bug != "no_normalise":
        p = p / ls[:, None]
    o = (p @ k) if bug == "k_for_v" else (p @ v)
    if bug == "lse_no_log":
        lse = np.where(empty, -np.inf, ms + ls)
    elif bug == "lse_log2":
        lse = np.where(empty, -np.inf, ms + np.log2(ls))
    elif bug == "lse_no_max":
        lse = np.where(empty, -np.inf, np.log(ls))
    else:
        lse = np.where(empty, -np.inf, ms + np.log(ls))
    return o, lse


DENSE_BUGS = ["no_scale", "strict_causal", "top_left_causal", "off_by_one_causal", "exp_sign",
              "no_normalise", "k_for_v", "lse_no_log", "lse_log2", "lse_no_max"]


def _fails_some(checks, fn):
    for c in checks:
        try:
            c(fn)
        except (AssertionError, ValueError, IndexError):
            return True
    return False


@pytest.mark.parametrize("bug", DENSE_BUGS)
def test_dense_mutant_caught(bug):
    # the unmutated copy passes, the mutant does not
    assert not _fails_some(ALL_CHECKS, lambda q, k, v, s, c: _attn_variant(q, k, v, s, c, None))
    assert _fails_some(ALL_CHECKS, lambda q, k, v, s, c: _attn_variant(q, k, v, s, c, bug))


def _online_variant(q, k, v, scale, causal, bm, bn, bug):
    """A copy of the oracle's tiled attention (per-tile states folded with the
    log-sum-exp combination) with one planted mistake."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    lq, lk = q.shape[0], k.shape[0]
    vis_all = (np.arange(lk)[None, :] <= (lk - lq) + np.arange(lq)[:, None]) if causal \
        else np.ones((lq, lk), dtype=bool)

    def tile_state(r0, r1, c0, c1):
        vis = vis_all[r0:r1, c0:c1]
        s = np.where(vis, scale * (q[r0:r1] @ k[c0:c1].T), -np.inf)
        m = s.max(axis=1)
        m_ref = np.where(np.isfinite(m), m, 0.0)
        e = np.where(vis, np.exp(s - m_ref[:, None]), 0.0)
        o = e @ v[c0:c1]
        if bug == "normalise_each_tile":
            o = o / np.where(e.sum(axis=1) > 0, e.sum(axis=1), 1.0)[:, None]
        return m, e.sum(axis=1), o

    def combine(a, b):
        (ma, la, oa), (mb, lb, ob) = a, b
        m = np.maximum(ma, mb)
        m_ref = np.where(np.isfinite(m), m, 0.0)
        if bug == "weight_sign":
            wa = np.where(np.isfinite(ma), np.exp(m_ref - ma), 0.0)
        else:
            wa = np.where(np.isfinite(ma), np.exp(ma - m_ref), 0.0)
        wb = np.where(np.isfinite(mb), np.exp(mb - m_ref), 0.0)
        l = (la + wb * lb) if bug == "no_rescale_l" else (wa * la + wb * lb)
        o = (oa + wb[:, None] * ob) if bug == "no_rescale_o" else (wa[:, None] * oa + wb[:, None] * ob)
        return m, l, o

    out = np.zeros((lq, v.shape[1]))
    lse = np.full(lq, -np.inf)
    for r0 in range(0, lq, bm):
        r1 = min(r0 + bm, lq)
        state = (np.full(r1 - r0, -np.inf), np.zeros(r1 - r0), np.zeros((r1 - r0, v.shape[1])))
        for c0 in range(0, lk, bn):
            state = combine(state, tile_state(r0, r1, c0, min(c0 + bn, lk)))
        m, l, acc = state
        done = l > 0
        out[r0:r1] = np.where(done[:, None], acc / np.where(done, l, 1.0)[:, None], 0.0)
        lse[r0:r1] = np.where(done, m + np.log(np.where(done, l, 1.0)), -np.inf)
    return out, lse


@pytest.mark.parametrize("bug", ["weight_sign", "no_rescale_l", "no_rescale_o", "normalise_each_tile"])
def test_online_mutant_caught(bug):
    fn = lambda q, k, v, s, c: _online_variant(q, k, v, s, c, 2, 3, None)  # noqa: E731
    assert not _fails_some(ALL_CHECKS, fn)
    mut = lambda q, k, v, s, c: _online_variant(q, k, v, s, c, 2, 3, bug)  # noqa: E731
    assert _fails_some(ALL_CHECKS, mut)


def _gather_variant(pool, block_tables, seq_lens, block_size=16, bug=None):
    import torch
    tables = np.asarray(block_tables.tolist() if hasattr(block_tables, "tolist") else block_tables)
    lens = [int(x) for x in (seq_lens.tolist() if hasattr(seq_lens, "tolist") else seq_lens)]
    out = []
    for b in range(tables.shape[0]):
        n = lens[b]
        tok = np.arange(n)
        if bug == "logical_not_physical":
            phys = tok // block_size
        elif bug == "slot_block_swapped":
            phys = tables[b][tok % tables.shape[1]]
        elif bug == "next_block":
            phys = tables[b][np.minimum(tok // block_size + 1, tables.shape[1] - 1)]
        else:
            phys = tables[b][tok // block_size]
        slot = (tok // block_size) % block_size if bug == "slot_block_swapped" else tok % block_size
        if isinstance(pool, torch.Tensor):
            rows = pool[torch.from_numpy(phys), :, torch.from_numpy(slot), :]
            out.append(rows.permute(1, 0, 2).contiguous())
        else:
            out.append(np.ascontiguousarray(np.transpose(np.asarray(pool)[phys, :, slot, :], (1, 0, 2))))
    return out


@pytest.mark.parametrize("bug", ["logical_not_physical", "slot_block_swapped", "next_block"])
def test_gather_mutant_caught(bug):
    checks = [check_paging_fixture, check_gather_contiguous]
    assert not _fails_some(checks, lambda *a: _gather_variant(*a))
    assert _fails_some(checks, lambda *a: _gather_variant(*a, bug=bug))


def _merge_variant(o_parts, lse_parts, bug):
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)
    empty = ~np.isfinite(m)
    ms = np.where(empty, 0.0, m)
    if bug == "linear_weights":
        w = np.where(np.isfinite(lse_parts), lse_parts - ms[None] + 1.0, 0.0)
    elif bug == "weight_sign":
        w = np.where(np.isfinite(lse_parts), np.exp(ms[None] - lse_parts), 0.0)
    else:
        w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - ms[None]), 0.0)
    ws = w.sum(axis=0)
    wss = np.where(empty, 1.0, ws)
    o = (w[..., None] * o_parts).sum(axis=0)
    if bug != "no_divide":
        o = o / wss[..., None]
    o = np.where(empty[..., None], 0.0, o)
    lse = np.where(empty, -np.inf, ms + (0.0 if bug == "lse_max_only" else np.log(wss)))
    return o, lse


@pytest.mark.parametrize("bug", ["linear_weights", "weight_sign", "no_divide", "lse_max_only"])
def test_merge_mutant_caught(bug):
    def split_check(merge):
        check_split_merge(oracle.split_partials, merge, 5, 300, True)

    checks = [check_merge_closed_forms, split_check]
    assert not _fails_some(checks, lambda o, l: _merge_variant(o, l, None))
    assert _fails_some(checks, lambda o, l: _merge_variant(o, l, bug))


def _split_variant(q, k, v, scale, causal, num_splits, block_size=16, bug=None):
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    lq, lk = q.shape[0], k.shape[0]
    vis = oracle.causal_visibility(lq, lk) if causal else np.ones((lq, lk), dtype=bool)
    op = np.zeros((num_splits, lq, v.shape[1]))
    lp = np.full((num_splits, lq), -np.inf)
    for p, (a, b) in enumerate(oracle.split_ranges(lk, num_splits, block_size)):
        if b <= a:
            continue
        if bug == "overlap":
            a = max(0, a - 1)
        if bug == "local_causal":
            sub = oracle.causal_visibility(lq, b - a) if causal else None
        else:
            sub = vis[:, a:b]
        op[p], lp[p] = oracle.masked_attention(q, k[a:b], v[a:b], scale, sub)
    return op, lp


@pytest.mark.parametrize("bug", ["overlap", "local_causal"])
def test_split_mutant_caught(bug):
    def run(bugv):
        def chk(_):
            check_split_merge(lambda *a: _split_variant(*a, bug=bugv), oracle.lse_merge, 5, 300, True)
        return chk

    assert not _fails_some([run(None)], None)
    assert _fails_some([run(bug)], None)


def _append_variant(k_pool, v_pool, block_tables, seq_lens, k_new, v_new, block_size=16,
                    bug=None):
    tables = np.asarray(block_tables, dtype=np.int64)
    lens = np.asarray(seq_lens, dtype=np.int64)
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    n_new = k_new.shape[2]
    for b in range(tables.shape[0]):
        for t in range(n_new):
            p = int(lens[b]) + t if bug == "position_after_len" else int(lens[b]) - n_new + t
            if p < 0 or (bug == "first_token_dropped" and t == 0):
                continue
            blk = p % block_size if bug == "slot_block_swapped" else p // block_size
            phys = blk if bug == "logical_not_physical" else int(tables[b][blk])
            if phys < 0 or phys >= k_out.shape[0]:
                continue
            slot = p // block_size if bug == "slot_block_swapped" else p % block_size
            slot = min(slot, block_size - 1)
            k_out[phys, :, slot, :] = k_new[b, :, t, :]
            v_out[phys, :, slot, :] = (k_new if bug == "k_for_v" else v_new)[b, :, t, :]
    return k_out, v_out


APPEND_BUGS = ["position_after_len", "first_token_dropped", "slot_block_swapped",
               "logical_not_physical", "k_for_v"]


@pytest.mark.parametrize("bug", APPEND_BUGS)
def test_append_mutant_caught(bug, monkeypatch):
    from tests import test_kv_cache as pins

    def variant(*a, **kw):
        return _append_variant(*a, bug=bug, **kw)

    monkeypatch.setattr(oracle, "paged_append", variant)
    checks = [pins.test_append_places_tokens_as_the_paging_figure_draws_them,
              pins.test_append_then_gather_round_trip,
              pins.test_append_in_pieces_equals_append_at_once,
              pins.test_append_skips_negative_positions]
    caught = 0
    for chk in checks:
        try:
            chk()
        except (AssertionError, IndexError, ValueError):
            caught += 1
    assert caught > 0


def _copy_variant(k_pool, v_pool, src, dst, bug=None):
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    for s, d in zip(src, dst):
        if bug == "reversed":
            s, d = d, s
        k_out[int(d)] = k_pool[int(s)]
        if bug != "k_only":
            v_out[int(d)] = v_pool[int(s)]
    return k_out, v_out


@pytest.mark.parametrize("bug", ["reversed", "k_only"])
def test_copy_mutant_caught(bug, monkeypatch):
    from tests import test_kv_cache as pins
    monkeypatch.setattr(oracle, "copy_blocks", lambda *a: _copy_variant(*a, bug=bug))
    with pytest.raises(AssertionError):
        pins.test_copy_blocks_preserves_what_a_rewritten_table_reads()


# ------------------------------------------------------------------ fp8 ---

def _encode_variant(x, bug):
    from oracle import fp8 as f
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x.astype(np.float64))
    if bug != "no_clamp":
        a = np.minimum(a, f.E4M3_MAX)
    hi = np.minimum(np.searchsorted(f._POS_VALS, a, side="left"), len(f._POS_VALS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - f._POS_VALS[lo]
    d_hi = f._POS_VALS[hi] - a
    if bug == "ties_away":
        pick_hi = d_hi <= d_lo
    elif bug == "truncate":
        pick_hi = d_hi == 0
    else:
        pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (f._POS_CODES[hi] % 2 == 0))
    if bug == "no_clamp":
        pick_hi = pick_hi | (a > f.E4M3_MAX)
        mag = np.where(a > f.E4M3_MAX, 0x7F, np.where(pick_hi, f._POS_CODES[hi], f._POS_CODES[lo]))
    else:
        mag = np.where(pick_hi, f._POS_CODES[hi], f._POS_CODES[lo])
    return (mag | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


@pytest.mark.parametrize("bug", ["ties_away", "truncate", "no_clamp"])
def test_fp8_encode_mutant_caught(bug, monkeypatch):
    from oracle import fp8 as f
    from tests import test_fp8_oracle as pins
    var = lambda x: _encode_variant(x, bug)  # noqa: E731
    monkeypatch.setattr(oracle, "e4m3_encode", var)
    monkeypatch.setattr(f, "e4m3_encode", var)
    checks = [pins.test_encode_matches_library_on_values_and_ties,
              pins.test_encode_clamps_out_of_range,
              pins.test_append_fresh_blocks_error_bound_and_max_code]
    caught = 0
    for chk in checks:
        try:
            chk()
        except AssertionError:
            caught += 1
    assert caught > 0


def _append_fp8_variant(bug):
    from oracle import fp8 as f

    def run(k_codes, k_scale, v_codes, v_scale, block_tables, seq_lens, k_new, v_new,
            block_size=16):
        tables = np.asarray(block_tables, dtype=np.int64)
        lens = np.asarray(seq_lens, dtype=np.int64)
        out = []
        for codes, scale, new in ((k_codes, k_scale, k_new), (v_codes, v_scale, v_new)):
            c = np.array(codes, dtype=np.uint8, copy=True)
            s = np.array(scale, dtype=np.float32, copy=True)
            x = np.asarray(new, dtype=np.float32)
            n_new = x.shape[2]
            for b in range(tables.shape[0]):
                first = max(int(lens[b]) - n_new, 0)
                last = int(lens[b])
                p = first
                while p < last:
                    lb = p // block_size
                    s0 = p - lb * block_size
                    s1 = min(last - lb * block_size, block_size)
                    phys = int(tables[b][lb])
                    t0 = lb * block_size + s0 - (int(lens[b]) - n_new)
                    for h in range(c.shape[1]):
                        vals = x[b, h, t0:t0 + (s1 - s0)]
                        amax = np.float32(np.max(np.abs(vals)))
                        s_old = np.float32(0) if (s0 == 0 and bug != "stale_scale") else s[phys, h]
                        cand = np.float32(amax / np.float32(448))
                        s_new = cand if bug == "scale_shrinks" else max(s_old, cand)
                        if s_new > s_old and s0 > 0 and bug != "no_reencode":
                            old = f.e4m3_decode(c[phys, h, :s0]).astype(np.float32)
                            c[phys, h, :s0] = f.e4m3_encode((old * s_old) / s_new)
                        c[phys, h, s0:s1] = f.e4m3_encode(vals / s_new) if s_new > 0 else 0
                        s[phys, h] = s_new
                    p = lb * block_size + s1
            out += [c, s]
        return tuple(out)
    return run


@pytest.mark.parametrize("bug", ["stale_scale", "scale_shrinks", "no_reencode"])
def test_fp8_append_mutant_caught(bug, monkeypatch):
    from tests import test_fp8_oracle as pins
    monkeypatch.setattr(oracle, "quantize_append", _append_fp8_variant(bug))
    checks = [pins.test_append_fresh_blocks_error_bound_and_max_code,
              pins.test_append_exact_on_representable_values,
              pins.test_append_in_pieces_equals_at_once_while_scale_stands,
              pins.test_append_growing_scale_reencodes_old_slots,
              pins.test_append_at_slot_zero_ignores_a_stale_scale,
              pins.test_append_all_zero_block_has_zero_scale]
    caught = 0
    for chk in checks:
        try:
            chk()
        except AssertionError:
            caught += 1
    assert caught > 0


def test_fp8_append_variant_without_bug_passes(monkeypatch):
    """The mutant harness itself: with no planted bug every pin passes."""
    from tests import test_fp8_oracle as pins
    monkeypatch.setattr(oracle, "quantize_append", _append_fp8_variant(None))
    pins.test_append_fresh_blocks_error_bound_and_max_code()
    pins.test_append_growing_scale_reencodes_old_slots()
    pins.test_append_at_slot_zero_ignores_a_stale_scale()
