"""Plain float64 definitions of what the attention library computes.

TEST INFRASTRUCTURE ONLY (see the package docstring): slow, obviously correct,
materialises the full score matrix S and probability matrix P. Inputs may be
torch CPU tensors (float32 / bfloat16) or numpy arrays; every stored value is
upcast exactly to float64 before any arithmetic, so input quantisation is not
counted as error.

Readings taken where the pages leave a step open (each one is listed with its
reason in the design notes of the repository):
  * scale: S = scale * Q K^T with ``scale`` an explicit argument ([P2] §一 gives
    1/sqrt(d_k); the [P1] §2.2 pseudocode omits it).
  * causal alignment when the query count Lq is below the key count Lk:
    bottom-right, i.e. query t sits at absolute position Lk - Lq + t and sees
    keys 0 .. Lk - Lq + t. This is what "verify prefix + K drafts in one
    forward" ([P3], speculative-sampling item) needs; with Lq == Lk it is the
    usual lower triangle.
  * a row that sees no key has output 0 and log-sum-exp -inf.
  * log-sum-exp uses the natural logarithm.
"""

import numpy as np

try:  # torch is only used to read bfloat16 tensors exactly
    import torch
except ImportError:  # pragma: no cover
    torch = None


def _f64(x):
    """Exact float64 copy of a torch tensor or array-like."""
    if torch is not None and isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _i64(x):
    if torch is not None and isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.int64).numpy()
    return np.asarray(x, dtype=np.int64)


def causal_visibility(lq, lk):
    """Boolean [lq, lk]: True where query t may attend key j.

    Bottom-right alignment: key j is visible to query t iff j <= (lk - lq) + t.
    """
    t = np.arange(lq)[:, None]
    j = np.arange(lk)[None, :]
    return j <= (lk - lq) + t


def masked_attention(q, k, v, scale, visible, return_p=False):
    """softmax(scale * q k^T restricted to ``visible``) v, in float64.

    Standard attention as [P1] §2.1 and [P2] §一 define it: the whole score
    matrix S is formed, the softmax is taken row by row over the visible keys
    (subtracting the row maximum first, which leaves the softmax unchanged),
    and the normalised P multiplies V.

    q [Lq, D], k [Lk, D], v [Lk, Dv]; ``visible`` bool [Lq, Lk] or None (all).
    Returns (o [Lq, Dv], lse [Lq]) and, if ``return_p``, also P [Lq, Lk].
    Rows with no visible key give o = 0, lse = -inf, P = 0.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    lq, lk = q.shape[0], k.shape[0]
    s = scale * (q @ k.T)
    if visible is None:
        visible = np.ones((lq, lk), dtype=bool)
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=1) if lk > 0 else np.full(lq, -np.inf)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    p = np.where(visible, np.exp(s - m_safe[:, None]), 0.0)
    l = p.sum(axis=1)
    l_safe = np.where(empty, 1.0, l)
    p = p / l_safe[:, None]
    o = p @ v
    lse = np.where(empty, -np.inf, m_safe + np.log(l_safe))
    if return_p:
        return o, lse, p
    return o, lse


def dense_attention(q, k, v, scale, causal, return_p=False):
    """One (batch, head) of exact attention, causal mask bottom-right aligned."""
    lq, lk = np.shape(q)[0], np.shape(k)[0]
    vis = causal_visibility(lq, lk) if causal else None
    return masked_attention(q, k, v, scale, vis, return_p=return_p)


def prefill(q, k, v, scale, causal, heads=None):
    """Exact attention over [B, H, L, D] tensors, one (b, h) at a time.

    Returns (o [B, H, Lq, D] float64, lse [B, H, Lq] float64). ``heads`` may be
    an iterable of (b, h) pairs to evaluate only those (other entries are NaN),
    for sampled checks at full size.
    """
    B, H, lq, D = q.shape
    o = np.full((B, H, lq, v.shape[3]), np.nan)
    lse = np.full((B, H, lq), np.nan)
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in pairs:
        o[b, h], lse[b, h] = dense_attention(q[b, h], k[b, h], v[b, h], scale, causal)
    return o, lse


def block_state(q, k, v, scale, visible):
    """Softmax state of one set of keys: (m, l, O) per query row.

    m is the largest visible score of the row, l the sum of exp(s - m) over
    its visible keys and O the sum of exp(s - m) v_j (unnormalised). A row
    that sees none of these keys has m = -inf, l = 0, O = 0. The softmax
    result over the keys is O / l with log-sum-exp m + log l.
    """
    s = scale * (q @ k.T)
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=1) if k.shape[0] > 0 else np.full(q.shape[0], -np.inf)
    m_ref = np.where(np.isfinite(m), m, 0.0)
    e = np.where(visible, np.exp(s - m_ref[:, None]), 0.0)
    return m, e.sum(axis=1), e @ v


def combine_states(a, b):
    """The state over the union of two disjoint key sets.

    With M = max(m_a, m_b), both states are brought to the common reference:
    l = e^(m_a - M) l_a + e^(m_b - M) l_b and O likewise, since
    exp(s - m_a) e^(m_a - M) = exp(s - M) for every key. The operation is
    associative and commutative, which is why the key range may be cut into
    tiles and folded in any grouping ([P1] §2.2: the tiled result equals the
    softmax over the whole row). A side with m = -inf contributes 0, and
    -inf - (-inf) is never formed.
    """
    (ma, la, oa), (mb, lb, ob) = a, b
    m = np.maximum(ma, mb)
    m_ref = np.where(np.isfinite(m), m, 0.0)
    wa = np.where(np.isfinite(ma), np.exp(ma - m_ref), 0.0)
    wb = np.where(np.isfinite(mb), np.exp(mb - m_ref), 0.0)
    return m, wa * la + wb * lb, wa[:, None] * oa + wb[:, None] * ob


def online_softmax_attention(q, k, v, scale, causal, bm, bn):
    """Tiled attention: per-tile softmax states folded into a running state.

    The tiling of [P1] §2.2: Q is cut into row blocks of ``bm`` rows (the outer
    loop, as FlashAttention-2 orders it in [P3]) and K, V into blocks of ``bn``
    keys. Each key block's own state (block_state) is folded into the row
    block's running state with combine_states, in key order, starting from the
    empty state (m = -inf, l = 0, O = 0); O / l is formed once per row block
    after its last key block. Returns (o [Lq, Dv], lse [Lq]); rows that see no
    key give o = 0, lse = -inf.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    lq, lk = q.shape[0], k.shape[0]
    vis_all = causal_visibility(lq, lk) if causal else np.ones((lq, lk), dtype=bool)
    out = np.zeros((lq, v.shape[1]))
    lse = np.full(lq, -np.inf)
    for r0 in range(0, lq, bm):
        r1 = min(r0 + bm, lq)
        state = (np.full(r1 - r0, -np.inf), np.zeros(r1 - r0), np.zeros((r1 - r0, v.shape[1])))
        for c0 in range(0, lk, bn):
            c1 = min(c0 + bn, lk)
            tile = block_state(q[r0:r1], k[c0:c1], v[c0:c1], scale, vis_all[r0:r1, c0:c1])
            state = combine_states(state, tile)
        m, l, acc = state
        done = l > 0
        out[r0:r1] = np.where(done[:, None], acc / np.where(done, l, 1.0)[:, None], 0.0)
        lse[r0:r1] = np.where(done, m + np.log(np.where(done, l, 1.0)), -np.inf)
    return out, lse


def paged_gather(pool, block_tables, seq_lens, block_size=16):
    """Read each sequence's cache rows back through its block table.

    PagedAttention as [P1] §3.2, [P3] and [P4] describe it: the cache is a pool
    of fixed-size physical blocks (16 tokens), and each sequence owns a table
    mapping its logical block n to a physical block id. Token t of sequence b
    lives in logical block t // block_size, slot t % block_size, i.e. at
    pool[block_tables[b][t // block_size], :, t % block_size, :].

    pool [num_blocks, H, block_size, D] (any dtype); returns a list with one
    array per sequence, [H, seq_len_b, D], holding exactly the pool's values
    (same dtype, no arithmetic). Table entries past the last used block and
    slots past seq_len are never read.
    """
    tables = _i64(block_tables)
    lens = _i64(seq_lens)
    is_torch = torch is not None and isinstance(pool, torch.Tensor)
    out = []
    for b in range(tables.shape[0]):
        n = int(lens[b])
        tok = np.arange(n)
        phys = tables[b][tok // block_size]
        slot = tok % block_size
        if is_torch:
            rows = pool[torch.from_numpy(phys), :, torch.from_numpy(slot), :]  # [n, H, D]
            out.append(rows.permute(1, 0, 2).contiguous())
        else:
            rows = np.asarray(pool)[phys, :, slot, :]
            out.append(np.ascontiguousarray(np.transpose(rows, (1, 0, 2))))
    return out


def paged_attention(q, k_pool, v_pool, block_tables, seq_lens, scale, causal,
                    block_size=16, heads=None):
    """Attention of q [B, Hq, Lq, D] over each sequence's paged K/V.

    The key count of sequence b is seq_lens[b] and includes the Lq new tokens,
    so with ``causal`` query t sits at position seq_len - Lq + t (bottom-right).
    The pools hold Hkv heads with Hq a multiple of Hkv; query head hq attends KV
    head hq // (Hq // Hkv) (grouped-query attention; Hq == Hkv is ordinary
    multi-head attention). Returns (o [B, Hq, Lq, D], lse [B, Hq, Lq]) in
    float64; with ``heads`` only those (b, hq) pairs are evaluated (others NaN).
    """
    B, H, lq, D = q.shape
    hkv = k_pool.shape[1]
    if H % hkv != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    group = H // hkv
    o = np.full((B, H, lq, v_pool.shape[3]), np.nan)
    lse = np.full((B, H, lq), np.nan)
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    bsel = sorted({b for b, _ in pairs})
    tables = _i64(block_tables)
    lens = _i64(seq_lens)
    for b in bsel:
        kc = paged_gather(k_pool, tables[b:b + 1], lens[b:b + 1], block_size)[0]
        vc = paged_gather(v_pool, tables[b:b + 1], lens[b:b + 1], block_size)[0]
        for bb, h in pairs:
            if bb != b:
                continue
            o[b, h], lse[b, h] = dense_attention(q[b, h], kc[h // group], vc[h // group], scale,
                                                 causal)
    return o, lse


def paged_attention_varlen(q, cu_q_lens, k_pool, v_pool, block_tables, seq_lens, scale, causal,
                           block_size=16, seqs=None):
    """Ragged-batch paged attention: sequence b brings its own query count.

    q [total_q, H, D] is token-major: sequence b owns tokens cu_q_lens[b] ..
    cu_q_lens[b+1]-1, its t-th new token at position seq_lens[b] - q_len_b + t
    (bottom-right causal, as in paged_attention). Each sequence is an ordinary
    paged attention problem of its own ([P1] §3.2 cache, [P1] §2.1 attention);
    continuous batching only packs them into one call. The pools may hold fewer
    heads than q (grouped-query: query head h reads KV head h // (H / Hkv)).
    Returns (o [total_q, H, D], lse [total_q, H]) in float64; with ``seqs`` only
    those sequences are evaluated (the other rows are NaN).
    """
    cu = _i64(cu_q_lens)
    tables = _i64(block_tables)
    lens = _i64(seq_lens)
    total, H, _ = q.shape
    hkv = k_pool.shape[1]
    if H % hkv != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    group = H // hkv
    o = np.full((total, H, v_pool.shape[3]), np.nan)
    lse = np.full((total, H), np.nan)
    for b in (range(len(cu) - 1) if seqs is None else seqs):
        a, e = int(cu[b]), int(cu[b + 1])
        if e == a:
            continue
        kc = paged_gather(k_pool, tables[b:b + 1], lens[b:b + 1], block_size)[0]
        vc = paged_gather(v_pool, tables[b:b + 1], lens[b:b + 1], block_size)[0]
        for h in range(H):
            o[a:e, h], lse[a:e, h] = dense_attention(q[a:e, h], kc[h // group], vc[h // group],
                                                     scale, causal)
    return o, lse


def split_ranges(seq_len, num_splits, block_size=16):
    """Token ranges of the split-KV partition of one sequence.

    FlashDecoding ([P3]) cuts the key range along the sequence into pieces
    handled independently. Reading used here: the sequence's nb = ceil(seq_len
    / block_size) blocks are cut into ``num_splits`` contiguous, block-aligned
    ranges of ceil(nb / num_splits) blocks; the last ranges may be short or
    empty. Returns a list of (start, end) token indices.
    """
    nb = -(-seq_len // block_size)
    per = -(-nb // num_splits) if nb > 0 else 0
    out = []
    for p in range(num_splits):
        b0 = min(p * per, nb)
        b1 = min((p + 1) * per, nb)
        out.append((min(b0 * block_size, seq_len), min(b1 * block_size, seq_len)))
    return out


def split_partials(q, k, v, scale, causal, num_splits, block_size=16):
    """Per-split normalised outputs and log-sum-exps for one (batch, head).

    q [Lq, D], k/v [Lk, D] (the whole key range of the sequence). Split p
    attends only keys in its range (with the same absolute causal mask as the
    unsplit problem) and returns its own softmax-normalised o_p and lse_p; an
    empty or fully masked range gives o_p = 0, lse_p = -inf.
    Returns (o_parts [S, Lq, Dv], lse_parts [S, Lq]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    lq, lk = q.shape[0], k.shape[0]
    vis = causal_visibility(lq, lk) if causal else np.ones((lq, lk), dtype=bool)
    o_parts = np.zeros((num_splits, lq, v.shape[1]))
    lse_parts = np.full((num_splits, lq), -np.inf)
    for p, (a, b) in enumerate(split_ranges(lk, num_splits, block_size)):
        if b > a:
            o_parts[p], lse_parts[p] = masked_attention(q, k[a:b], v[a:b], scale, vis[:, a:b])
    return o_parts, lse_parts


def lse_merge(o_parts, lse_parts):
    """Combine split-KV partials into the full result.

    Each partial p holds softmax-normalised o_p and lse_p = log(sum of exp of
    its scores). The full softmax is recovered by weighting o_p with
    exp(lse_p - M) for M = max_p lse_p and dividing by the sum of the weights;
    the full lse is M + log(sum of weights). This is the same rescaling that
    merges two key blocks in the online-softmax recurrence of [P1] §2.2, done
    once across splits -- the cross-block reduction FlashDecoding ([P3])
    describes. Rows whose partials are all -inf give o = 0, lse = -inf.

    o_parts [S, ..., D], lse_parts [S, ...] -> (o [..., D], lse [...]).
    """
    o_parts = _f64(o_parts)
    lse_parts = _f64(lse_parts)
    m = lse_parts.max(axis=0)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - m_safe[None]), 0.0)
    wsum = w.sum(axis=0)
    wsum_safe = np.where(empty, 1.0, wsum)
    o = (w[..., None] * o_parts).sum(axis=0) / wsum_safe[..., None]
    o = np.where(empty[..., None], 0.0, o)
    lse = np.where(empty, -np.inf, m_safe + np.log(wsum_safe))
    return o, lse
