"""GPU parity: the HIP kernels, called through the C ABI, against the CPU oracle.

Tolerances (max abs error over all compared elements):
  * float32 prefill: 1e-5 on O.
  * bfloat16 paths: 2e-2 on O (fp32 accumulation; the output rounding to bf16
    alone is up to 2^-8 |O|), 1e-3 on the float32 log-sum-exp.
  * block-table indexing (gather): bit-exact; paged outputs bit-identical under
    a permutation of the physical blocks.
Full-size workloads are checked on every (batch, head) pair against the
oracle, in the launch configuration the benchmark times (tiling must equal the
one-shot softmax on every row, [P1] §2.2); the oracle takes seconds to tens of
seconds per workload on the host cores.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from workloads import (C1, C2, C3, C4, C5, PagedInputs, PagedSpec, PrefillSpec, paged_inputs,
                       permute_pool, prefill_inputs)

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 2e-2
TOL_LSE = 1e-3


@pytest.fixture(scope="module")
def api():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import attention_tiled_qk_amd as m
    return m


def say(msg):
    print(msg, flush=True)


def to_dev(*ts):
    return [t.cuda() for t in ts]


def max_err(gpu, ref, pairs=None):
    g = gpu.detach().double().cpu().numpy()
    if pairs is None:
        return float(np.abs(g - ref).max())
    return max(float(np.abs(g[b, h] - ref[b, h]).max()) for b, h in pairs)


def lse_err(gpu, ref, pairs=None):
    g = gpu.detach().double().cpu().numpy()
    if pairs is not None:
        g = np.stack([g[b, h] for b, h in pairs])
        ref = np.stack([ref[b, h] for b, h in pairs])
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(g), fin)
    return float(np.abs(g[fin] - ref[fin]).max()) if fin.any() else 0.0


def test_device_report():
    p = torch.cuda.get_device_properties(0)
    say(f"device: {p.name} arch={getattr(p, 'gcnArchName', '?')} CUs={p.multi_processor_count} "
        f"mem={p.total_memory / 2**30:.0f} GiB")


# ------------------------------------------------------------------ prefill ---

PREFILL_SMALL = [
    PrefillSpec("f32_c1_shape", 1, 1, 128, 64, "f32", True, 1),
    PrefillSpec("f32_ragged_full_d128", 2, 2, 200, 128, "f32", False, 11),
    PrefillSpec("f32_L1", 1, 3, 1, 64, "f32", True, 12),
    PrefillSpec("f32_ragged_causal_d64", 1, 2, 333, 64, "f32", True, 13),
    PrefillSpec("bf16_ragged_causal", 2, 3, 300, 128, "bf16", True, 21),
    PrefillSpec("bf16_ragged_full", 2, 3, 300, 128, "bf16", False, 22),
    PrefillSpec("bf16_L1", 1, 2, 1, 128, "bf16", True, 23),
    PrefillSpec("bf16_L17_d64", 1, 2, 17, 64, "bf16", True, 24),
    PrefillSpec("bf16_513_full_d64", 1, 1, 513, 64, "bf16", False, 25),
    PrefillSpec("bf16_129_causal", 3, 2, 129, 128, "bf16", True, 26),
    PrefillSpec("bf16_1024_causal", 1, 2, 1024, 128, "bf16", True, 27),
]


@pytest.mark.parametrize("spec", PREFILL_SMALL, ids=lambda s: s.name)
def test_prefill_small(api, spec):
    say(f"prefill {spec}")
    q, k, v = prefill_inputs(spec)
    ref_o, ref_lse = oracle.prefill(q, k, v, spec.scale, spec.causal)
    dq, dk, dv = to_dev(q, k, v)
    o, lse = api.attn_prefill(dq, dk, dv, causal=spec.causal, scale=spec.scale, return_lse=True)
    torch.cuda.synchronize()
    tol = TOL_F32 if spec.dtype == "f32" else TOL_BF16
    e = max_err(o, ref_o)
    el = lse_err(lse, ref_lse)
    say(f"  max|dO|={e:.3e} (tol {tol}) max|dlse|={el:.3e}")
    assert e <= tol
    assert el <= (TOL_F32 if spec.dtype == "f32" else TOL_LSE)


def test_prefill_c1_exact_config(api):
    q, k, v = prefill_inputs(C1)
    ref, _ = oracle.prefill(q, k, v, C1.scale, C1.causal)
    o = api.attn_prefill(*to_dev(q, k, v), causal=True, scale=C1.scale)
    e = max_err(o, ref)
    say(f"c1: max|dO|={e:.3e}")
    assert e <= TOL_F32


@pytest.mark.parametrize("spec", [C2, C3], ids=["c2", "c3"])
def test_prefill_full_size(api, spec):
    say(f"full-size {spec.name}, every (batch, head) against the oracle")
    q, k, v = prefill_inputs(spec)
    o, lse = api.attn_prefill(*to_dev(q, k, v), causal=spec.causal, scale=spec.scale,
                              return_lse=True)
    torch.cuda.synchronize()
    ref_o, ref_lse = oracle.prefill(q, k, v, spec.scale, spec.causal)
    e = max_err(o, ref_o)
    el = lse_err(lse, ref_lse)
    say(f"  max|dO|={e:.3e} max|dlse|={el:.3e}")
    assert e <= TOL_BF16 and el <= TOL_LSE
    assert torch.isfinite(o.float()).all()


def _prefill_vs_oracle(api, q, k, v, scale, causal, tol, lse_tol=TOL_LSE):
    ref_o, ref_lse = oracle.prefill(q, k, v, scale, causal)
    o, lse = api.attn_prefill(*to_dev(q, k, v), causal=causal, scale=scale, return_lse=True)
    torch.cuda.synchronize()
    e = max_err(o, ref_o)
    el = lse_err(lse, ref_lse)
    say(f"  max|dO|={e:.3e} max|dlse|={el:.3e}")
    assert torch.isfinite(o.float()).all()
    assert e <= tol and el <= lse_tol


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_growing_scores(api, causal):
    """Scores that keep growing along the keys: every query has a component of
    about 3 along d = 0 and key j one of 11 j, so a row's scores rise by about
    2.9 per key and its maximum outgrows the reference max (by 2^30 in the
    exponent) many times over the sequence."""
    g = torch.Generator().manual_seed(31)
    B, H, L, D = 1, 2, 700, 128
    q = torch.randn(B, H, L, D, generator=g)
    k = torch.randn(B, H, L, D, generator=g)
    v = torch.randn(B, H, L, D, generator=g)
    q[..., 0] += 3.0
    k[..., 0] += 11.0 * torch.arange(L, dtype=torch.float32)
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    _prefill_vs_oracle(api, q, k, v, 1.0 / math.sqrt(D), causal, TOL_BF16)


def test_prefill_late_outlier_key(api):
    """One key far above all others late in the sequence: every row that sees it
    must move its reference max there and rescale what it accumulated."""
    g = torch.Generator().manual_seed(32)
    B, H, L, D = 1, 2, 640, 128
    q = torch.randn(B, H, L, D, generator=g)
    k = torch.randn(B, H, L, D, generator=g)
    v = torch.randn(B, H, L, D, generator=g)
    q[..., 0] += 3.0
    k[:, :, 500, 0] = 2000.0
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    _prefill_vs_oracle(api, q, k, v, 1.0 / math.sqrt(D), True, TOL_BF16)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("scale", [-1.0 / math.sqrt(128), 0.0, 0.5])
def test_prefill_other_scales(api, scale, dtype):
    """Negative, zero and large scales (the reference max is taken over
    scale-signed scores; scale 0 gives the mean of the visible values), on the
    bf16 matrix-core kernel and on the float32 kernel (1e-5 on O and lse)."""
    spec = PrefillSpec("scales", 1, 2, 300, 128, dtype, True, 33)
    q, k, v = prefill_inputs(spec)
    if dtype == "f32":
        _prefill_vs_oracle(api, q, k, v, scale, True, TOL_F32, 1e-5)
    else:
        _prefill_vs_oracle(api, q, k, v, scale, True, TOL_BF16)


def test_prefill_deterministic(api):
    q, k, v = to_dev(*prefill_inputs(PrefillSpec("d", 2, 2, 300, 128, "bf16", True, 5)))
    o1 = api.attn_prefill(q, k, v)
    o2 = api.attn_prefill(q, k, v)
    assert torch.equal(o1, o2)


# -------------------------------------------------------------------- paged ---

def _paged(lens, q_len, H=3, D=128, seed=0, extra=4, prefix=0, poison=True):
    """Paged inputs with explicit lengths (NaN in every slot no table may read)."""
    g = torch.Generator().manual_seed(seed)
    nb = [-(-n // 16) for n in lens]
    own = [n - prefix for n in nb]
    total = prefix + sum(own) + extra
    perm = torch.randperm(total, generator=g)
    width = max(nb) + 2
    tables = torch.full((len(lens), width), -1, dtype=torch.int32)
    pos = prefix
    for b in range(len(lens)):
        row = torch.cat([perm[:prefix], perm[pos:pos + own[b]]])
        pos += own[b]
        tables[b, :row.numel()] = row.to(torch.int32)
    k_pool = torch.randn(total, H, 16, D, generator=g).to(torch.bfloat16)
    v_pool = torch.randn(total, H, 16, D, generator=g).to(torch.bfloat16)
    q = torch.randn(len(lens), H, q_len, D, generator=g).to(torch.bfloat16)
    lens_t = torch.tensor(lens, dtype=torch.int32)
    if poison:
        readable = torch.zeros(total, 16, dtype=torch.bool)
        for b, n in enumerate(lens):
            for t in range(n):
                readable[int(tables[b, t // 16]), t % 16] = True
        idx = (~readable).nonzero(as_tuple=True)
        k_pool[idx[0], :, idx[1], :] = float("nan")
        v_pool[idx[0], :, idx[1], :] = float("nan")
    return PagedInputs(q, k_pool, v_pool, tables, lens_t)


def _run_paged(api, inp, splits, causal=True, scale=None):
    D = inp.q.shape[3]
    scale = scale if scale is not None else 1.0 / math.sqrt(D)
    dq, dk, dv, dt, dl = to_dev(inp.q, inp.k_pool, inp.v_pool, inp.block_tables, inp.seq_lens)
    o, lse = api.attn_paged_decode(dq, dk, dv, dt, dl, causal=causal, scale=scale,
                                   num_splits=splits, return_lse=True)
    torch.cuda.synchronize()
    return o, lse


PAGED_CASES = [
    ((1, 16, 17, 100, 257, 1000), 1),
    ((5, 16, 17, 100, 257, 1000), 5),
    ((16, 17, 33, 100, 257, 1000), 16),
    ((31, 48, 49), 3),
]


@pytest.mark.parametrize("lens,q_len", PAGED_CASES)
@pytest.mark.parametrize("splits", [1, 2, 3, 16, 0])
@pytest.mark.parametrize("causal", [True, False])
def test_paged_small(api, lens, q_len, splits, causal):
    say(f"paged lens={lens} q_len={q_len} splits={splits} causal={causal}")
    inp = _paged(lens, q_len, seed=len(lens) * 31 + q_len)
    scale = 1.0 / math.sqrt(128)
    ref_o, ref_lse = oracle.paged_attention(inp.q, inp.k_pool, inp.v_pool, inp.block_tables,
                                            inp.seq_lens, scale, causal)
    o, lse = _run_paged(api, inp, splits, causal)
    e = max_err(o, ref_o)
    el = lse_err(lse, ref_lse)
    say(f"  max|dO|={e:.3e} max|dlse|={el:.3e}")
    assert torch.isfinite(o.float()).all()
    assert e <= TOL_BF16 and el <= TOL_LSE


@pytest.mark.parametrize("splits", [1, 2, 0])
def test_paged_long_split_crosses_id_chunks(api, splits):
    """Splits longer than the 256 block ids the kernel stages at a time."""
    inp = _paged((4200, 9000, 300), 5, H=2, seed=41, extra=3)
    scale = 1.0 / math.sqrt(128)
    ref_o, ref_lse = oracle.paged_attention(inp.q, inp.k_pool, inp.v_pool, inp.block_tables,
                                            inp.seq_lens, scale, True)
    o, lse = _run_paged(api, inp, splits)
    e = max_err(o, ref_o)
    say(f"  splits={splits} max|dO|={e:.3e}")
    assert torch.isfinite(o.float()).all()
    assert e <= TOL_BF16 and lse_err(lse, ref_lse) <= TOL_LSE


@pytest.mark.parametrize("scale", [-1.0 / math.sqrt(128), 0.0])
def test_paged_other_scales(api, scale):
    inp = _paged((5, 100, 257, 1000), 5, seed=42)
    ref_o, ref_lse = oracle.paged_attention(inp.q, inp.k_pool, inp.v_pool, inp.block_tables,
                                            inp.seq_lens, scale, True)
    o, lse = _run_paged(api, inp, 3, True, scale)
    assert torch.isfinite(o.float()).all()
    assert max_err(o, ref_o) <= TOL_BF16 and lse_err(lse, ref_lse) <= TOL_LSE


GQA_CASES = [(8, 1), (4, 4), (16, 1), (2, 5), (5, 3)]


def _gqa_inputs(lens, q_len, hkv, group, seed):
    inp = _paged(lens, q_len, H=hkv, seed=seed)
    g = torch.Generator().manual_seed(seed + 1)
    q = torch.randn(len(lens), hkv * group, q_len, 128, generator=g).to(torch.bfloat16)
    return PagedInputs(q, inp.k_pool, inp.v_pool, inp.block_tables, inp.seq_lens)


@pytest.mark.parametrize("group,q_len", GQA_CASES)
@pytest.mark.parametrize("splits", [1, 3, 0])
def test_paged_gqa(api, group, q_len, splits):
    say(f"gqa group={group} q_len={q_len} splits={splits}")
    inp = _gqa_inputs((q_len, 17, 100, 257, 1000), q_len, 2, group, seed=50 + group)
    scale = 1.0 / math.sqrt(128)
    ref_o, ref_lse = oracle.paged_attention(inp.q, inp.k_pool, inp.v_pool, inp.block_tables,
                                            inp.seq_lens, scale, True)
    o, lse = _run_paged(api, inp, splits)
    e = max_err(o, ref_o)
    say(f"  max|dO|={e:.3e}")
    assert torch.isfinite(o.float()).all()
    assert e <= TOL_BF16 and lse_err(lse, ref_lse) <= TOL_LSE


def _reorder(inp, order):
    """The same sequences in another batch order (same pools and blocks)."""
    idx = torch.tensor(order)
    return PagedInputs(inp.q[idx].contiguous(), inp.k_pool, inp.v_pool,
                       inp.block_tables[idx].contiguous(), inp.seq_lens[idx].contiguous())


# Batches with tied lengths, at and past the 64 sequences that the kernel's
# longest-first order takes (one length per lane), with long splits (the order
# is used) and short ones (batch order).
LPT_CASES = [
    ((300, 1000, 17, 1000, 300, 5, 1000, 64), 1, 2, 1),
    (tuple(16 + (i * 37) % 1100 // 50 * 50 for i in range(64)), 2, 1, 1),
    (tuple(16 + (i * 37) % 1100 // 50 * 50 for i in range(65)), 1, 1, 1),
    ((40, 900, 900, 40, 2000, 41), 3, 2, 2),
]


@pytest.mark.parametrize("lens,q_len,hkv,splits", LPT_CASES)
def test_paged_longest_first_order(api, lens, q_len, hkv, splits):
    """Each sequence's output does not depend on where it stands in the batch
    (the kernel maps launch positions to sequences by length rank), and it
    matches the oracle."""
    say(f"longest-first: B={len(lens)} q_len={q_len} hkv={hkv} splits={splits}")
    group = 2
    inp = _gqa_inputs(lens, q_len, hkv, group, seed=len(lens) + 7)
    scale = 1.0 / math.sqrt(128)
    o1, l1 = _run_paged(api, inp, splits)
    order = list(range(len(lens)))[::-1]
    order = order[1::2] + order[0::2]
    o2, l2 = _run_paged(api, _reorder(inp, order), splits)
    inv = torch.empty(len(order), dtype=torch.long)
    inv[torch.tensor(order)] = torch.arange(len(order))
    assert torch.equal(o1, o2[inv.cuda()]) and torch.equal(l1, l2[inv.cuda()])
    ref_o, ref_lse = oracle.paged_attention(inp.q, inp.k_pool, inp.v_pool, inp.block_tables,
                                            inp.seq_lens, scale, True)
    e = max_err(o1, ref_o)
    say(f"  max|dO|={e:.3e}")
    assert e <= TOL_BF16 and lse_err(l1, ref_lse) <= TOL_LSE


def test_paged_gqa_bit_identical_under_block_permutation(api):
    inp = _gqa_inputs((5, 100, 257, 1000), 2, 2, 4, seed=60)
    o1, l1 = _run_paged(api, inp, 3)
    perm = permute_pool(inp, 4321)
    o2, l2 = _run_paged(api, perm, 3)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_paged_gqa_full_size(api):
    from workloads import C4G
    inp = paged_inputs(C4G)
    o, lse = _run_paged(api, inp, C4G.num_splits, True, C4G.scale)
    ref_o, ref_lse = oracle.paged_attention(inp.q, inp.k_pool, inp.v_pool, inp.block_tables,
                                            inp.seq_lens, C4G.scale, True)
    e = max_err(o, ref_o)
    say(f"  gqa full size, all pairs: max|dO|={e:.3e}")
    assert torch.isfinite(o.float()).all()
    assert e <= TOL_BF16 and lse_err(lse, ref_lse) <= TOL_LSE


def _run_paged_prefill(api, inp, causal=True, scale=None):
    D = inp.q.shape[3]
    scale = scale if scale is not None else 1.0 / math.sqrt(D)
    dq, dk, dv, dt, dl = to_dev(inp.q, inp.k_pool, inp.v_pool, inp.block_tables, inp.seq_lens)
    o, lse = api.attn_paged_prefill(dq, dk, dv, dt, dl, causal=causal, scale=scale,
                                    return_lse=True)
    torch.cuda.synchronize()
    return o, lse


PAGED_PREFILL_CASES = [
    ((300, 1000, 2500), 300, 128),
    ((77, 77, 200), 77, 128),
    ((1, 16, 64, 65), 1, 128),
    ((513, 4097), 513, 64),
]


@pytest.mark.parametrize("lens,q_len,D", PAGED_PREFILL_CASES)
@pytest.mark.parametrize("causal", [True, False])
def test_paged_prefill(api, lens, q_len, D, causal):
    say(f"paged prefill lens={lens} q_len={q_len} D={D} causal={causal}")
    inp = _paged(lens, q_len, H=3, D=D, seed=70 + q_len)
    scale = 1.0 / math.sqrt(D)
    ref_o, ref_lse = oracle.paged_attention(inp.q, inp.k_pool, inp.v_pool, inp.block_tables,
                                            inp.seq_lens, scale, causal)
    o, lse = _run_paged_prefill(api, inp, causal, scale)
    e = max_err(o, ref_o)
    el = lse_err(lse, ref_lse)
    say(f"  max|dO|={e:.3e} max|dlse|={el:.3e}")
    assert torch.isfinite(o.float()).all()
    assert e <= TOL_BF16 and el <= TOL_LSE


def test_paged_prefill_bit_identical_under_block_permutation(api):
    inp = _paged((300, 1000), 200, H=2, seed=80)
    o1, l1 = _run_paged_prefill(api, inp)
    perm = permute_pool(inp, 77)
    o2, l2 = _run_paged_prefill(api, perm)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("nb_big", [65535, 65600, 131200])
def test_paged_prefill_large_pool_matches_compact_pool(api, nb_big):
    """A pool of 65535 blocks of 8 heads x 16 x 128 is 32 KiB short of 2^31 bytes
    (one buffer range for the whole pool, per-lane offsets up to its top); 65600
    blocks pass 2^31 bytes and take the kernel's other addressing path (a buffer
    range per 1 KiB piece); 131200 blocks pass 2^31 elements. The same problem laid out in such a pool -- blocks near its
    end, every other slot NaN -- and in a compact pool must give bit-identical
    outputs and log-sum-exps."""
    H, D = 8, 128
    lens = (300, 1000)
    q_len = 64
    need = [(n + 15) // 16 for n in lens]
    g = torch.Generator().manual_seed(91)
    total = sum(need)
    k_small = torch.randn(total, H, 16, D, generator=g).to(torch.bfloat16)
    v_small = torch.randn(total, H, 16, D, generator=g).to(torch.bfloat16)
    q = torch.randn(len(lens), H, q_len, D, generator=g).to(torch.bfloat16)
    width = max(need)
    tab_small = torch.full((len(lens), width), -1, dtype=torch.int32)
    tab_big = torch.full((len(lens), width), -1, dtype=torch.int32)
    # big-pool ids: the last blocks of the pool for the first sequence, a spread
    # across the pool (ending near its top) for the second
    big_ids = list(range(nb_big - need[0], nb_big)) + [100 + 1000 * i for i in range(need[1])]
    c = 0
    for b, n in enumerate(need):
        for j in range(n):
            tab_small[b, j] = c
            tab_big[b, j] = big_ids[c]
            c += 1
    dev = torch.device("cuda")
    k_big = torch.full((nb_big, H, 16, D), float("nan"), dtype=torch.bfloat16, device=dev)
    v_big = torch.full((nb_big, H, 16, D), float("nan"), dtype=torch.bfloat16, device=dev)
    idx = torch.tensor(big_ids, dtype=torch.long, device=dev)
    k_sd, v_sd = k_small.to(dev), v_small.to(dev)
    # tail slots past each sequence's end stay NaN in the big pool as well
    for b, n in enumerate(lens):
        last = sum(need[:b + 1]) - 1
        if n % 16:
            k_sd[last, :, n % 16:] = float("nan")
            v_sd[last, :, n % 16:] = float("nan")
    k_big[idx] = k_sd
    v_big[idx] = v_sd
    seq = torch.tensor(lens, dtype=torch.int32, device=dev)
    qd = q.to(dev)
    o1, l1 = api.attn_paged_prefill(qd, k_sd, v_sd, tab_small.to(dev), seq, causal=True, return_lse=True)
    o2, l2 = api.attn_paged_prefill(qd, k_big, v_big, tab_big.to(dev), seq, causal=True, return_lse=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o1.float()).all()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    del k_big, v_big
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_past_2pow31_elements(api, dtype):
    """Q, K, V and O of B=1, H=16400, L=1024, D=128 hold 2^31 + 2^21 elements
    each (4.3 GB in bf16, 8.6 GB in float32); head 16384 is the first to start
    at element 2^31. The heads on both sides of that boundary, the first and
    the last match the oracle: offsets are formed in 64 bits."""
    B, H, L, D = 1, 16400, 1024, 128
    assert B * H * L * D > 2**31 and 16384 * L * D == 2**31
    dev = torch.device("cuda")
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator(device=dev).manual_seed(93)
    q, k, v = (torch.randn((B, H, L, D), device=dev, dtype=dt, generator=g) for _ in range(3))
    scale = 1.0 / math.sqrt(D)
    say(f"prefill {dtype} past 2^31 elements: B={B} H={H} L={L} D={D}")
    o, lse = api.attn_prefill(q, k, v, causal=True, scale=scale, return_lse=True)
    torch.cuda.synchronize()
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    lse_tol = TOL_LSE if dtype == "bf16" else TOL_F32
    for h in (0, 16383, 16384, H - 1):
        ref_o, ref_lse = oracle.dense_attention(q[0, h].cpu(), k[0, h].cpu(), v[0, h].cpu(), scale, True)
        e = float(np.abs(o[0, h].double().cpu().numpy() - ref_o).max())
        el = float(np.abs(lse[0, h].double().cpu().numpy() - ref_lse).max())
        say(f"  head {h}: max|dO|={e:.3e} max|dlse|={el:.3e}")
        assert e <= tol and el <= lse_tol
    del q, k, v, o, lse
    torch.cuda.empty_cache()


@pytest.mark.parametrize("q_len,splits", [(1, 0), (1, 1), (5, 16)])
def test_paged_decode_pool_past_2pow31_elements_matches_compact_pool(api, q_len, splits):
    """A pool of 131200 blocks of 8 heads x 16 x 128 holds more than 2^31
    elements (4.3 GB each for K and V); blocks from 131072 on start past
    element 2^31. The same problem laid out near the end of such a pool --
    every other slot NaN -- and in a compact pool must give bit-identical
    outputs and log-sum-exps."""
    H, D, nb_big = 8, 128, 131200
    assert nb_big * H * 16 * D > 2**31 and 131072 * H * 16 * D == 2**31
    lens = (300, 1000)
    need = [(n + 15) // 16 for n in lens]
    g = torch.Generator().manual_seed(94)
    total = sum(need)
    k_small = torch.randn(total, H, 16, D, generator=g).to(torch.bfloat16)
    v_small = torch.randn(total, H, 16, D, generator=g).to(torch.bfloat16)
    q = torch.randn(len(lens), H, q_len, D, generator=g).to(torch.bfloat16)
    width = max(need)
    tab_small = torch.full((len(lens), width), -1, dtype=torch.int32)
    tab_big = torch.full((len(lens), width), -1, dtype=torch.int32)
    # the first sequence in the pool's last blocks (all past element 2^31), the
    # second spread across the pool, its last blocks past the boundary too
    big_ids = (list(range(nb_big - need[0], nb_big)) + [2000 * i + 7 for i in range(need[1] - 4)]
               + [131072 + 20 * j for j in range(4)])
    assert max(big_ids) < nb_big and len(set(big_ids)) == len(big_ids)
    assert sum(i >= 131072 for i in big_ids[need[0]:]) > 0
    c = 0
    for b, n in enumerate(need):
        for j in range(n):
            tab_small[b, j] = c
            tab_big[b, j] = big_ids[c]
            c += 1
    dev = torch.device("cuda")
    k_sd, v_sd = k_small.to(dev), v_small.to(dev)
    for b, n in enumerate(lens):
        last = sum(need[:b + 1]) - 1
        if n % 16:
            k_sd[last, :, n % 16:] = float("nan")
            v_sd[last, :, n % 16:] = float("nan")
    k_big = torch.full((nb_big, H, 16, D), float("nan"), dtype=torch.bfloat16, device=dev)
    v_big = torch.full((nb_big, H, 16, D), float("nan"), dtype=torch.bfloat16, device=dev)
    idx = torch.tensor(big_ids, dtype=torch.long, device=dev)
    k_big[idx] = k_sd
    v_big[idx] = v_sd
    seq = torch.tensor(lens, dtype=torch.int32, device=dev)
    qd = q.to(dev)
    say(f"paged decode, pool of {nb_big} blocks, q_len={q_len} splits={splits}")
    o1, l1 = api.attn_paged_decode(qd, k_sd, v_sd, tab_small.to(dev), seq, causal=True,
                                   num_splits=splits, return_lse=True)
    o2, l2 = api.attn_paged_decode(qd, k_big, v_big, tab_big.to(dev), seq, causal=True,
                                   num_splits=splits, return_lse=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o1.float()).all()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    scale = 1.0 / math.sqrt(D)
    ref_o, ref_lse = oracle.paged_attention(q, k_sd.cpu(), v_sd.cpu(), tab_small, torch.tensor(lens),
                                            scale, True)
    e = max_err(o2, ref_o)
    say(f"  max|dO|={e:.3e}")
    assert e <= TOL_BF16 and lse_err(l2, ref_lse) <= TOL_LSE
    del k_big, v_big
    torch.cuda.empty_cache()


def test_paged_prefill_fresh_sequence_matches_prefill(api):
    """A chunk that is the whole sequence (q_len == seq_len) is ordinary causal
    prefill of the gathered K/V: same kernel arithmetic, same result bits."""
    n = 700
    inp = _paged((n,), n, H=2, seed=81, poison=False)
    kc = oracle.paged_gather(inp.k_pool, inp.block_tables, inp.seq_lens)[0][None]
    vc = oracle.paged_gather(inp.v_pool, inp.block_tables, inp.seq_lens)[0][None]
    o_paged, _ = _run_paged_prefill(api, inp)
    o_pre = api.attn_prefill(*to_dev(inp.q, kc, vc), causal=True)
    assert torch.equal(o_paged, o_pre)


def test_paged_prefill_full_size(api):
    from workloads import CPF
    inp = paged_inputs(CPF)
    o, lse = _run_paged_prefill(api, inp, True, CPF.scale)
    ref_o, ref_lse = oracle.paged_attention(inp.q, inp.k_pool, inp.v_pool, inp.block_tables,
                                            inp.seq_lens, CPF.scale, True)
    e = max_err(o, ref_o)
    say(f"  chunked prefill full size, all pairs: max|dO|={e:.3e}")
    assert torch.isfinite(o.float()).all()
    assert e <= TOL_BF16 and lse_err(lse, ref_lse) <= TOL_LSE


def _run_varlen(api, inp, qlens, q, causal=True, scale=None):
    cu = torch.tensor(np.concatenate([[0], np.cumsum(qlens)]), dtype=torch.int32)
    D = q.shape[2]
    scale = scale if scale is not None else 1.0 / math.sqrt(D)
    dq, dk, dv, dt, dl, dc = to_dev(q, inp.k_pool, inp.v_pool, inp.block_tables, inp.seq_lens, cu)
    o, lse = api.attn_paged_prefill_varlen(dq, dk, dv, dt, dl, dc, max(qlens), causal=causal,
                                           scale=scale, return_lse=True)
    torch.cuda.synchronize()
    return o, lse, cu


VARLEN_CASES = [
    ((300, 1000, 2500, 64, 700), (300, 1, 130, 0, 700), 128),
    ((16, 17, 4097, 33), (16, 2, 257, 33), 64),
]


@pytest.mark.parametrize("lens,qlens,D", VARLEN_CASES)
@pytest.mark.parametrize("causal", [True, False])
def test_paged_prefill_varlen(api, lens, qlens, D, causal):
    say(f"varlen prefill lens={lens} qlens={qlens} D={D} causal={causal}")
    inp = _paged(lens, 1, H=3, D=D, seed=90 + D)
    g = torch.Generator().manual_seed(91)
    q = torch.randn(sum(qlens), 3, D, generator=g).to(torch.bfloat16)
    scale = 1.0 / math.sqrt(D)
    o, lse, cu = _run_varlen(api, inp, qlens, q, causal, scale)
    ref_o, ref_lse = oracle.paged_attention_varlen(q, cu, inp.k_pool, inp.v_pool,
                                                   inp.block_tables, inp.seq_lens, scale, causal)
    e = max_err(o, ref_o)
    el = lse_err(lse, ref_lse)
    say(f"  max|dO|={e:.3e} max|dlse|={el:.3e}")
    assert torch.isfinite(o.float()).all()
    assert e <= TOL_BF16 and el <= TOL_LSE


@pytest.mark.parametrize("group,D", [(4, 128), (8, 128), (2, 64)])
def test_paged_prefill_gqa(api, group, D):
    """Ragged chunked prefill over grouped-query pools (query head h reads KV
    head h // group)."""
    lens, qlens = (300, 1000, 77, 513), (300, 1, 77, 200)
    inp = _paged(lens, 1, H=2, D=D, seed=97 + group)
    g = torch.Generator().manual_seed(98)
    q = torch.randn(sum(qlens), 2 * group, D, generator=g).to(torch.bfloat16)
    say(f"gqa prefill group={group} D={D} lens={lens} qlens={qlens}")
    o, lse, cu = _run_varlen(api, inp, qlens, q)
    ref_o, ref_lse = oracle.paged_attention_varlen(q, cu, inp.k_pool, inp.v_pool,
                                                   inp.block_tables, inp.seq_lens,
                                                   1 / math.sqrt(D), True)
    e, el = max_err(o, ref_o), lse_err(lse, ref_lse)
    say(f"  max|dO|={e:.3e} max|dlse|={el:.3e}")
    assert e <= TOL_BF16 and el <= TOL_LSE


def test_paged_prefill_gqa_equals_repeated_kv_heads_bitwise(api):
    """The grouped call gives the bits of the multi-head call on a pool whose
    KV heads are repeated: the same kernel arithmetic, other K/V addresses."""
    group = 4
    inp = _paged((400, 900), 1, H=2, seed=99, poison=False)
    g = torch.Generator().manual_seed(100)
    qlens = [400, 130]
    q = torch.randn(sum(qlens), 2 * group, 128, generator=g).to(torch.bfloat16)
    o1, l1, _ = _run_varlen(api, inp, qlens, q)
    rep = PagedInputs(inp.q, inp.k_pool.repeat_interleave(group, dim=1).contiguous(),
                      inp.v_pool.repeat_interleave(group, dim=1).contiguous(), inp.block_tables,
                      inp.seq_lens)
    o2, l2, _ = _run_varlen(api, rep, qlens, q)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_paged_prefill_varlen_equal_lengths_bit_identical(api):
    """Equal query counts: the ragged call gives attn_paged_prefill's bits."""
    inp = _paged((300, 1000, 200), 200, H=2, seed=92)
    o1, l1 = _run_paged_prefill(api, inp)
    B, H, lq, D = inp.q.shape
    packed = inp.q.permute(0, 2, 1, 3).contiguous().reshape(B * lq, H, D)
    o2, l2, _ = _run_varlen(api, inp, [lq] * B, packed)
    assert torch.equal(o2.reshape(B, lq, H, D).permute(0, 2, 1, 3), o1)
    assert torch.equal(l2.reshape(B, lq, H).permute(0, 2, 1), l1)


def test_paged_prefill_varlen_mixed_batch_full_size(api):
    """A continuous-batching step at the 13B shape: 4 sequences bring a
    512-token prompt chunk and 4 bring one decode token, 40 heads, 4096 cached
    keys each; every sequence against the oracle."""
    from workloads import CPF
    inp = paged_inputs(CPF)
    qlens = [512, 1, 512, 1, 512, 1, 512, 1]
    g = torch.Generator().manual_seed(93)
    q = torch.randn(sum(qlens), CPF.H, CPF.D, generator=g).to(torch.bfloat16)
    o, lse, cu = _run_varlen(api, inp, qlens, q, True, CPF.scale)
    ref_o, ref_lse = oracle.paged_attention_varlen(q, cu, inp.k_pool, inp.v_pool,
                                                   inp.block_tables, inp.seq_lens, CPF.scale,
                                                   True)
    e = float(np.abs(o.double().cpu().numpy() - ref_o).max())
    el = float(np.abs(lse.double().cpu().numpy() - ref_lse).max())
    say(f"  mixed batch max|dO|={e:.3e} max|dlse|={el:.3e}")
    assert e <= TOL_BF16 and el <= TOL_LSE


def test_paged_d64(api):
    inp = _paged((7, 70, 300), 5, D=64, seed=3)
    ref_o, _ = oracle.paged_attention(inp.q, inp.k_pool, inp.v_pool, inp.block_tables,
                                      inp.seq_lens, 0.125, True)
    o, _ = _run_paged(api, inp, 2, True, 0.125)
    assert max_err(o, ref_o) <= TOL_BF16


@pytest.mark.parametrize("splits", [1, 16])
def test_paged_bit_identical_under_block_permutation(api, splits):
    inp = _paged((5, 100, 257, 1000), 5, seed=9)
    o1, l1 = _run_paged(api, inp, splits)
    perm = permute_pool(inp, 1234)
    assert not torch.equal(perm.block_tables, inp.block_tables)
    o2, l2 = _run_paged(api, perm, splits)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_paged_split_invariance(api):
    inp = _paged((2000, 3000, 4096), 5, seed=10)
    o1, _ = _run_paged(api, inp, 1)
    for s in [2, 7, 16, 64]:
        o2, _ = _run_paged(api, inp, s)
        d = (o1.float() - o2.float()).abs().max().item()
        say(f"  S=1 vs S={s}: {d:.3e}")
        assert d <= TOL_BF16


def test_paged_full_query_matches_prefill(api):
    """q_len == seq_len over a fresh paged sequence equals causal prefill."""
    n = 16
    inp = _paged((n,), n, H=2, seed=4, poison=False)
    kc = oracle.paged_gather(inp.k_pool, inp.block_tables, inp.seq_lens)[0][None]
    vc = oracle.paged_gather(inp.v_pool, inp.block_tables, inp.seq_lens)[0][None]
    o_paged, _ = _run_paged(api, inp, 1)
    o_pre = api.attn_prefill(*to_dev(inp.q, kc, vc), causal=True)
    d = (o_paged.float() - o_pre.float()).abs().max().item()
    say(f"  paged vs prefill: {d:.3e}")
    assert d <= TOL_BF16


def test_paged_shared_prefix(api):
    inp = _paged((40, 64, 90, 33), 5, seed=12, prefix=2)
    ref_o, _ = oracle.paged_attention(inp.q, inp.k_pool, inp.v_pool, inp.block_tables,
                                      inp.seq_lens, 1 / math.sqrt(128), True)
    o, _ = _run_paged(api, inp, 3)
    assert max_err(o, ref_o) <= TOL_BF16


# ------------------------------------------------------------------- gather ---

def test_gather_bit_exact(api):
    inp = _paged((1, 16, 17, 100, 257), 1, seed=2, extra=6)
    ml = 300
    out = api.attn_paged_gather(*to_dev(inp.k_pool, inp.block_tables, inp.seq_lens), ml)
    ref = oracle.paged_gather(inp.k_pool, inp.block_tables, inp.seq_lens)
    got = out.cpu()
    for b, n in enumerate(inp.seq_lens.tolist()):
        assert torch.equal(got[b, :, :n].view(torch.int16), ref[b].view(torch.int16))
        assert torch.all(got[b, :, n:] == 0)


def test_gather_paging_figure(api):
    """The pool of the paging figure in [P1] section 3.2, A:[0,1,5,7,8], B:[2,9]."""
    H, D = 2, 64
    pool = torch.arange(11 * H * 16 * D, dtype=torch.float32).reshape(11, H, 16, D)
    pool = (pool % 251).to(torch.bfloat16)
    tables = torch.tensor([[0, 1, 5, 7, 8], [2, 9, -1, -1, -1]], dtype=torch.int32)
    lens = torch.tensor([70, 20], dtype=torch.int32)
    out = api.attn_paged_gather(*to_dev(pool, tables, lens), 80).cpu()
    ref = oracle.paged_gather(pool, tables, lens)
    assert torch.equal(out[0, :, :70], ref[0]) and torch.equal(out[1, :, :20], ref[1])


# -------------------------------------------------------------------- merge ---

def _count_bad_entries(tables, lens, min_len, num_blocks):
    """Host count, entry by entry, of what attn_paged_check_tables reports."""
    width = len(tables[0])
    bad_len = bad_id = 0
    for row, n in zip(tables, lens):
        if n < min_len or n > 16 * width:
            bad_len += 1
        for j in range((min(max(n, 0), 16 * width) + 15) // 16):
            if not 0 <= row[j] < num_blocks:
                bad_id += 1
    return bad_len, bad_id


def test_check_tables_counts_out_of_range_entries(api):
    """The table check finds nothing wrong in a valid decode description, and
    counts each planted fault: ids past the pool or negative inside a
    sequence's range, lengths past the table or below q_len, a negative
    length. Padding past a sequence's blocks is not counted."""
    inp = paged_inputs(C4)
    nb = inp.k_pool.shape[0]
    tab = inp.block_tables.clone()
    lens = inp.seq_lens.clone()
    width = tab.shape[1]
    dev = torch.device("cuda")
    assert api.attn_paged_check_tables(tab.to(dev), lens.to(dev), nb) == (0, 0)
    assert _count_bad_entries(tab.tolist(), lens.tolist(), 1, nb) == (0, 0)
    tab[0, 0] = nb                              # one past the pool
    tab[1, (int(lens[1]) - 1) // 16] = -1       # the last block of a sequence
    tab[2, 3] = 1 << 30
    n3 = int(lens[3])
    tab[3, (n3 + 15) // 16:] = nb + 5           # padding: never read, not counted
    n4 = int(lens[4])
    lens[4] = 16 * width + 1                    # longer than the table: its -1 padding is read
    lens[5] = 0                                 # shorter than q_len = 1
    lens[6] = -7
    expect = _count_bad_entries(tab.tolist(), lens.tolist(), 1, nb)
    assert expect == (3, 3 + width - (n4 + 15) // 16)
    got = api.attn_paged_check_tables(tab.to(dev), lens.to(dev), nb)
    say(f"table check: {got} (host count {expect})")
    assert got == expect
    # with q_len 5 the length-0 sequence stays bad and nothing else changes
    assert api.attn_paged_check_tables(tab.to(dev), lens.to(dev), nb, min_len=5) == \
        _count_bad_entries(tab.tolist(), lens.tolist(), 5, nb)


def test_check_tables_mode_refuses_bad_tables(api, monkeypatch):
    """With the debugging switch on (ATTN_CHECK_TABLES=1), paged calls with valid
    tables give the unchecked results, and a table entry past the pool makes
    decode, prefill, append and gather raise before anything is launched. The
    pools passed are views of the first N blocks of N + 1, so even the refused
    id lies in allocated memory."""
    H, D = 4, 128
    lens = [100, 300]
    need = [(n + 15) // 16 for n in lens]
    N = sum(need)
    g = torch.Generator().manual_seed(95)
    dev = torch.device("cuda")
    k_all = torch.randn(N + 1, H, 16, D, generator=g).to(torch.bfloat16).to(dev)
    v_all = torch.randn(N + 1, H, 16, D, generator=g).to(torch.bfloat16).to(dev)
    k, v = k_all[:N], v_all[:N]
    q = torch.randn(2, H, 1, D, generator=g).to(torch.bfloat16).to(dev)
    tab = torch.full((2, max(need)), -1, dtype=torch.int32)
    c = 0
    for b, n in enumerate(need):
        for j in range(n):
            tab[b, j] = c
            c += 1
    seq = torch.tensor(lens, dtype=torch.int32, device=dev)
    ref = api.attn_paged_decode(q, k, v, tab.to(dev), seq)
    monkeypatch.setattr(api, "CHECK_TABLES", True)
    assert torch.equal(api.attn_paged_decode(q, k, v, tab.to(dev), seq), ref)
    bad = tab.clone()
    bad[1, 0] = N
    bad = bad.to(dev)
    assert api.attn_paged_check_tables(bad, seq, N) == (0, 1)
    with pytest.raises(ValueError, match="ATTN_CHECK_TABLES"):
        api.attn_paged_decode(q, k, v, bad, seq)
    with pytest.raises(ValueError, match="ATTN_CHECK_TABLES"):
        api.attn_paged_prefill(q, k, v, bad, seq)
    with pytest.raises(ValueError, match="ATTN_CHECK_TABLES"):
        api.attn_paged_gather(k, bad, seq, 320)
    # the append writes through the entry of each sequence's newest position:
    # -1 there places nothing (accepted), an id past the pool is refused
    last = (lens[1] - 1) // 16
    skip = tab.clone()
    skip[1, last] = -1
    assert api.attn_paged_check_append(skip.to(dev), seq, N, 1) == (0, 0)
    bad_app = tab.clone()
    bad_app[1, last] = N
    assert api.attn_paged_check_append(bad_app.to(dev), seq, N, 1) == (0, 1)
    with pytest.raises(ValueError, match="ATTN_CHECK_TABLES"):
        api.attn_paged_append(q, q, k, v, bad_app.to(dev), seq)
    # ragged prefill: offsets that run past the packed queries are refused
    qv = torch.randn(6, H, D, generator=g).to(torch.bfloat16).to(dev)
    cu_bad = torch.tensor([0, 4, 7], dtype=torch.int32, device=dev)
    with pytest.raises(ValueError, match="ATTN_CHECK_TABLES"):
        api.attn_paged_prefill_varlen(qv, k, v, tab.to(dev), seq, cu_bad, 4)
    # block copies: a destination past the pool is refused
    src = torch.tensor([0], dtype=torch.int32, device=dev)
    dst_bad = torch.tensor([N], dtype=torch.int32, device=dev)
    with pytest.raises(ValueError, match="ATTN_CHECK_TABLES"):
        api.attn_paged_copy_blocks(k, v, src, dst_bad)
    torch.cuda.synchronize()
    assert torch.equal(k_all[:N], k) and torch.isfinite(k_all.float()).all()
    assert torch.isfinite(v_all.float()).all()


def _count_append_faults(tables, lens, n_new, num_blocks):
    """Host count of what attn_paged_check_append reports: lengths outside
    [0, 16 * width] and written-through entries neither -1 nor in the pool."""
    width = len(tables[0])
    bad_len = bad_id = 0
    for row, n in zip(tables, lens):
        if n < 0 or n > 16 * width:
            bad_len += 1
        hi = min(n, 16 * width)
        lo = max(0, hi - n_new)
        for j in sorted({p // 16 for p in range(lo, hi)}):
            if not (row[j] == -1 or 0 <= row[j] < num_blocks):
                bad_id += 1
    return bad_len, bad_id


def test_check_append_counts_faults(api):
    """The append check agrees with a host count, entry by entry, on valid
    tables, -1 entries (accepted), ids past the pool and below -1 at written
    positions (counted), faults at positions the append does not write (not
    counted) and lengths past the table or negative."""
    g = torch.Generator().manual_seed(41)
    B, W, nb, n_new = 7, 12, 50, 20
    lens = torch.randint(1, 16 * W + 1, (B,), generator=g, dtype=torch.int32)
    tab = torch.randint(0, nb, (B, W), generator=g, dtype=torch.int32)
    dev = torch.device("cuda")
    assert api.attn_paged_check_append(tab.to(dev), lens.to(dev), nb, n_new) == (0, 0)
    tab[0, (int(lens[0]) - 1) // 16] = -1        # skipped: fine
    tab[1, (int(lens[1]) - 1) // 16] = nb        # written: counted
    tab[2, (int(lens[2]) - 1) // 16] = -2        # written: counted
    if int(lens[3]) > n_new + 16:
        tab[3, 0] = nb + 9                       # never written: not counted
    lens[4] = 16 * W + 3                         # past the table
    lens[5] = -1
    expect = _count_append_faults(tab.tolist(), lens.tolist(), n_new, nb)
    got = api.attn_paged_check_append(tab.to(dev), lens.to(dev), nb, n_new)
    say(f"append check: {got} (host count {expect})")
    assert got == expect and expect[0] == 2 and expect[1] >= 2


def test_check_ragged_and_ids(api):
    """The ragged-offset and id-list checks agree with host counts."""
    dev = torch.device("cuda")
    lens = torch.tensor([10, 3, 40, 8], dtype=torch.int32)
    cu = torch.tensor([0, 5, 8, 40, 44], dtype=torch.int32)
    assert api.attn_paged_check_ragged(cu.to(dev), lens.to(dev), 44, 32) == (0, 0)
    # sequence 2 brings 32 queries: more than max_q_len 31 (not its length 40)
    assert api.attn_paged_check_ragged(cu.to(dev), lens.to(dev), 44, 31) == (0, 1)
    # a total past the last offset
    assert api.attn_paged_check_ragged(cu.to(dev), lens.to(dev), 45, 32) == (1, 0)
    cu2 = torch.tensor([1, 5, 9, 7, 44], dtype=torch.int32)
    # cu[0] != 0, a decreasing step, sequence 1 with 4 queries over 3 keys
    assert api.attn_paged_check_ragged(cu2.to(dev), lens.to(dev), 44, 40) == (2, 2)
    src = torch.tensor([0, 5, -1, 9, 10], dtype=torch.int32)
    dst = torch.tensor([1, 2, 3, 10, 4], dtype=torch.int32)
    assert api.attn_paged_check_ids(src.to(dev), dst.to(dev), 10) == (2, 1)
    assert api.attn_paged_check_ids(dst.to(dev), dst.to(dev), 11) == (0, 0)


@pytest.mark.parametrize("S,D", [(1, 128), (3, 128), (16, 128), (1024, 128), (7, 64)])
def test_lse_merge(api, S, D):
    g = torch.Generator().manual_seed(S)
    B, H, ql = 2, 3, 5
    op = torch.randn(B, H, ql, S, D, generator=g)
    lp = torch.randn(B, H, ql, S, generator=g) * 3
    if S > 1:
        lp[0, 0, 0, 1] = -float("inf")
        lp[1, 2, 4, :] = -float("inf")
    ref_o, ref_l = oracle.lse_merge(op.permute(3, 0, 1, 2, 4).numpy(), lp.permute(3, 0, 1, 2).numpy())
    o32, l32 = api.attn_lse_merge(*to_dev(op, lp), out_dtype=torch.float32, return_lse=True)
    obf = api.attn_lse_merge(*to_dev(op, lp), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert max_err(o32, ref_o) <= TOL_F32
    assert max_err(obf, ref_o) <= TOL_BF16
    assert lse_err(l32, ref_l) <= TOL_F32


# ------------------------------------------------------ largest shapes ---

@pytest.mark.parametrize("causal", [True, False])
def test_paged_prefill_widest_table(api, causal):
    """A sequence of 32768 keys: the full 2048-entry table the paged prefill
    kernel stages in LDS, with a ragged 200-token chunk."""
    inp = _paged((32768,), 200, H=2, seed=95, extra=0, poison=False)
    assert inp.block_tables.shape[1] >= 2048
    tables = inp.block_tables[:, :2048].contiguous()
    ref_o, ref_lse = oracle.paged_attention(inp.q, inp.k_pool, inp.v_pool, tables, inp.seq_lens,
                                            1 / math.sqrt(128), causal)
    o, lse = api.attn_paged_prefill(*to_dev(inp.q, inp.k_pool, inp.v_pool, tables, inp.seq_lens),
                                    causal=causal, return_lse=True)
    torch.cuda.synchronize()
    e, el = max_err(o, ref_o), lse_err(lse, ref_lse)
    say(f"  32768 keys, causal={causal}: max|dO|={e:.3e} max|dlse|={el:.3e}")
    assert e <= TOL_BF16 and el <= TOL_LSE


def test_paged_decode_widest_query_and_most_splits(api):
    """q_len 16 (the column limit) with the largest explicit split count, 64."""
    inp = _paged((16, 40, 700, 3000), 16, H=2, seed=96)
    ref_o, ref_lse = oracle.paged_attention(inp.q, inp.k_pool, inp.v_pool, inp.block_tables,
                                            inp.seq_lens, 1 / math.sqrt(128), True)
    o, lse = _run_paged(api, inp, 64)
    e, el = max_err(o, ref_o), lse_err(lse, ref_lse)
    say(f"  q_len 16, S=64: max|dO|={e:.3e} max|dlse|={el:.3e}")
    assert e <= TOL_BF16 and el <= TOL_LSE


# ------------------------------------------------------ full-size paged ---

@pytest.mark.parametrize("spec", [C4, C5], ids=["c4", "c5"])
def test_paged_full_size(api, spec):
    say(f"full-size {spec.name}, every (sequence, head) against the oracle")
    inp = paged_inputs(spec)
    lens = inp.seq_lens.tolist()
    order = sorted(range(spec.B), key=lambda b: lens[b])
    bs = sorted({order[0], order[-1], order[len(order) // 2], 1 % spec.B})
    o, lse = _run_paged(api, inp, spec.num_splits, spec.causal, spec.scale)
    ref_o, ref_lse = oracle.paged_attention(inp.q, inp.k_pool, inp.v_pool, inp.block_tables,
                                            inp.seq_lens, spec.scale, spec.causal)
    e = max_err(o, ref_o)
    el = lse_err(lse, ref_lse)
    say(f"  all pairs: max|dO|={e:.3e} max|dlse|={el:.3e}")
    assert torch.isfinite(o.float()).all()
    assert e <= TOL_BF16 and el <= TOL_LSE
    # block-table indexing on the same pool, bit-exact, for the sampled sequences
    ml = max(lens[b] for b in bs)
    sel = torch.tensor(bs)
    out = api.attn_paged_gather(inp.k_pool.cuda(), inp.block_tables[sel].cuda(),
                                inp.seq_lens[sel].cuda(), ml).cpu()
    ref = oracle.paged_gather(inp.k_pool, inp.block_tables[sel], inp.seq_lens[sel])
    for i, b in enumerate(bs):
        assert torch.equal(out[i, :, :lens[b]].view(torch.int16), ref[i].view(torch.int16))
