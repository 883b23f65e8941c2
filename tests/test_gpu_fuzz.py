"""Seeded random-shape parity sweep over every attention entry point.

Each case draws its shape from a fixed seed (so a failure names a reproducible
case) across the supported ranges: prefill L from 1 to a few tiles plus ragged
tails, D in {64, 128}, causal or full, float32 or bfloat16; paged decode with
lengths from 1 up, q_len and grouped-query group sizes up to the 16-column
limit, explicit and automatic split counts; ragged chunked prefill; and the
FP8 cache. Outputs are compared with the oracle at the same tolerances as the
other parity tests (1e-5 fp32, 2e-2 bf16 on O; 1e-3 on the bf16 paths' lse).
"""

import math
import random

import numpy as np
import pytest
import torch

import oracle
from workloads import PagedSpec, paged_inputs, paged_inputs_fp8

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 2e-2
TOL_LSE = 1e-3
BS = 16


@pytest.fixture(scope="module")
def api():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import attention_tiled_qk_amd as m
    return m


def say(msg):
    print(msg, flush=True)


def _cmp(o, lse, ro, rl, tol):
    on = o.double().cpu().numpy()
    ln = lse.double().cpu().numpy()
    e = float(np.abs(on - ro).max())
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(ln), fin)
    el = float(np.abs(ln[fin] - rl[fin]).max()) if fin.any() else 0.0
    return e, el


@pytest.mark.parametrize("case", range(32))
def test_prefill_random_shapes(api, case):
    rnd = random.Random(1000 + case)
    dtype = "f32" if case % 4 == 3 else "bf16"
    D = rnd.choice([64, 128])
    L = rnd.choice([1, 2, 31, 63, 64, 65, 127, 129, 200, 257, 390, 511])
    B, H = rnd.randint(1, 3), rnd.randint(1, 4)
    causal = rnd.random() < 0.7
    scale = rnd.choice([1.0 / math.sqrt(D), 0.3, 0.05])
    say(f"case {case}: prefill {dtype} B={B} H={H} L={L} D={D} causal={causal} scale={scale:.3f}")
    g = torch.Generator().manual_seed(case)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    q, k, v = (torch.randn(B, H, L, D, generator=g).to(tdt) for _ in range(3))
    ro, rl = oracle.prefill(q, k, v, scale, causal)
    o, lse = api.attn_prefill(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale,
                              return_lse=True)
    torch.cuda.synchronize()
    e, el = _cmp(o, lse, ro, rl, None)
    say(f"  max|dO|={e:.3e} max|dlse|={el:.3e}")
    assert e <= (TOL_F32 if dtype == "f32" else TOL_BF16)
    assert el <= (1e-5 if dtype == "f32" else TOL_LSE)


@pytest.mark.parametrize("case", range(32))
def test_paged_decode_random_shapes(api, case):
    rnd = random.Random(2000 + case)
    D = rnd.choice([64, 128])
    hkv = rnd.randint(1, 4)
    group = rnd.choice([1, 1, 2, 4, 8])
    q_len = rnd.randint(1, 16 // group)
    B = rnd.randint(1, 5)
    hi = rnd.choice([20, 300, 1500])
    lo = rnd.randint(q_len, hi)
    splits = rnd.choice([0, 0, 1, 3, 7])
    causal = rnd.random() < 0.8
    spec = PagedSpec("fz", B, hkv, q_len, D, seed=3000 + case, len_lo=lo, len_hi=hi,
                     extra_blocks=rnd.randint(0, 3), poison=True, q_heads=hkv * group)
    inp = paged_inputs(spec)
    say(f"case {case}: paged D={D} Hkv={hkv} group={group} q_len={q_len} "
        f"lens={inp.seq_lens.tolist()} S={splits} causal={causal}")
    ro, rl = oracle.paged_attention(inp.q, inp.k_pool, inp.v_pool, inp.block_tables,
                                    inp.seq_lens, spec.scale, causal)
    o, lse = api.attn_paged_decode(inp.q.cuda(), inp.k_pool.cuda(), inp.v_pool.cuda(),
                                   inp.block_tables.cuda(), inp.seq_lens.cuda(), causal=causal,
                                   num_splits=splits, return_lse=True)
    torch.cuda.synchronize()
    e, el = _cmp(o, lse, ro, rl, None)
    say(f"  max|dO|={e:.3e} max|dlse|={el:.3e}")
    assert torch.isfinite(o.float()).all()
    assert e <= TOL_BF16 and el <= TOL_LSE


@pytest.mark.parametrize("case", range(24))
def test_paged_prefill_varlen_random(api, case):
    rnd = random.Random(4000 + case)
    D = rnd.choice([64, 128])
    H = rnd.randint(1, 3)
    B = rnd.randint(1, 5)
    lens = [rnd.randint(1, 700) for _ in range(B)]
    qlens = [rnd.choice([0, 1, rnd.randint(1, n)]) if n > 0 else 0 for n in lens]
    if sum(qlens) == 0:
        qlens[0] = 1
    causal = rnd.random() < 0.8
    sl = torch.tensor(lens, dtype=torch.int32)
    nb = [-(-n // BS) for n in lens]
    g = torch.Generator().manual_seed(6000 + case)
    total = sum(nb) + 2
    perm = torch.randperm(total, generator=g)
    tables = torch.full((B, max(nb)), -1, dtype=torch.int32)
    pos = 0
    for b in range(B):
        tables[b, :nb[b]] = perm[pos:pos + nb[b]].to(torch.int32)
        pos += nb[b]
    k_pool = torch.randn(total, H, BS, D, generator=g).to(torch.bfloat16)
    v_pool = torch.randn(total, H, BS, D, generator=g).to(torch.bfloat16)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(qlens)]), dtype=torch.int32)
    q = torch.randn(int(cu[-1]), H, D, generator=g).to(torch.bfloat16)
    say(f"case {case}: varlen D={D} H={H} lens={lens} qlens={qlens} causal={causal}")
    ro, rl = oracle.paged_attention_varlen(q, cu, k_pool, v_pool, tables, sl, 1 / math.sqrt(D),
                                           causal)
    o, lse = api.attn_paged_prefill_varlen(q.cuda(), k_pool.cuda(), v_pool.cuda(), tables.cuda(),
                                           sl.cuda(), cu.cuda(), max(qlens), causal=causal,
                                           return_lse=True)
    torch.cuda.synchronize()
    e, el = _cmp(o, lse, ro, rl, None)
    say(f"  max|dO|={e:.3e} max|dlse|={el:.3e}")
    assert e <= TOL_BF16 and el <= TOL_LSE


@pytest.mark.parametrize("case", range(20))
def test_fp8_decode_random_shapes(api, case):
    rnd = random.Random(7000 + case)
    D = rnd.choice([64, 128])
    hkv = rnd.randint(1, 3)
    group = rnd.choice([1, 2, 4])
    q_len = rnd.randint(1, 16 // group)
    B = rnd.randint(1, 4)
    hi = rnd.choice([40, 500, 1200])
    spec = PagedSpec("fz8", B, hkv, q_len, D, seed=8000 + case, len_lo=rnd.randint(q_len, hi),
                     len_hi=hi, extra_blocks=2, poison=True, q_heads=hkv * group)
    inp = paged_inputs_fp8(spec)
    splits = rnd.choice([0, 1, 5])
    say(f"case {case}: fp8 D={D} Hkv={hkv} group={group} q_len={q_len} "
        f"lens={inp.seq_lens.tolist()} S={splits}")
    ro, rl = oracle.paged_attention_fp8(inp.q, inp.k_codes, inp.k_scale, inp.v_codes,
                                        inp.v_scale, inp.block_tables, inp.seq_lens, spec.scale,
                                        True)
    o, lse = api.attn_paged_decode_fp8(inp.q.cuda(), inp.k_codes.cuda(), inp.v_codes.cuda(),
                                       inp.k_scale.cuda(), inp.v_scale.cuda(),
                                       inp.block_tables.cuda(), inp.seq_lens.cuda(),
                                       num_splits=splits, return_lse=True)
    torch.cuda.synchronize()
    e, el = _cmp(o, lse, ro, rl, None)
    say(f"  max|dO|={e:.3e} max|dlse|={el:.3e}")
    assert e <= TOL_BF16 and el <= TOL_LSE
