"""GPU parity of the FP8 (E4M3, block-wise scaled) paged KV cache.

* attn_paged_append_fp8 decides integers (codes) from float32 arithmetic:
  codes and scales must equal the oracle's quantize_append bit for bit, over
  prefill chunks, decode steps whose values grow (re-encoding older slots)
  and blocks that start afresh over stale scales.
* attn_paged_copy_blocks_fp8 is bit-exact against the oracle's copy.
* attn_paged_decode_fp8 against the oracle's attention over the dequantised
  cache: max abs error 2e-2 on O (bf16 output, fp32 accumulation; the codes
  widen to bf16 exactly) and 1e-3 on the float32 log-sum-exp, like the other
  bf16 paths.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from workloads import C4F8, PagedSpec, paged_inputs_fp8

pytestmark = pytest.mark.gpu

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


def _tables(g, lens, nb, width):
    perm = torch.randperm(nb, generator=g)
    t = torch.full((len(lens), width), -1, dtype=torch.int32)
    pos = 0
    for b, n in enumerate(lens):
        m = -(-n // BS)
        t[b, :m] = perm[pos:pos + m].to(torch.int32)
        pos += m
    return t


def _stale(g, nb, H, D):
    codes = torch.randint(0, 0x7F, (nb, H, BS, D), generator=g, dtype=torch.uint8)
    scales = torch.rand((nb, H), generator=g) * 5.0
    return codes, scales


def _same(dev, ref):
    return np.array_equal(dev.cpu().numpy(), np.asarray(ref))


@pytest.mark.parametrize("D", [128, 64])
def test_append_fp8_bit_exact_over_a_growing_cache(api, D):
    g = torch.Generator().manual_seed(40 + D)
    H, width, nb = 4, 12, 64
    final = [150, 33, 97, 16, 180]
    prompt = [37, 16, 80, 1, 150]
    tables = _tables(g, final, nb, width)
    kc, ks = _stale(g, nb, H, D)
    vc, vs = _stale(g, nb, H, D)
    dk, dv, dks, dvs = kc.cuda(), vc.cuda(), ks.cuda(), vs.cuda()
    ref = (kc.numpy(), ks.numpy(), vc.numpy(), vs.numpy())
    dt = tables.cuda()

    def step(lens, n_new, mult):
        nonlocal ref
        kn = (torch.randn(len(lens), H, n_new, D, generator=g) * mult).to(torch.bfloat16)
        vn = (torch.randn(len(lens), H, n_new, D, generator=g) * mult).to(torch.bfloat16)
        sl = torch.tensor(lens, dtype=torch.int32)
        api.attn_paged_append_fp8(kn.cuda(), vn.cuda(), dk, dv, dks, dvs, dt, sl.cuda())
        ref = oracle.quantize_append(*ref, tables, sl, kn, vn)
        torch.cuda.synchronize()
        for dev, r, name in ((dk, ref[0], "k codes"), (dks, ref[1], "k scales"),
                             (dv, ref[2], "v codes"), (dvs, ref[3], "v scales")):
            assert _same(dev, r), name

    # prompt chunk (padded to the longest prompt; shorter ones start later)
    n0 = max(prompt)
    step(prompt, n0, 1.0)
    say(f"  D={D} prompt ok")
    lens = list(prompt)
    for s in range(30):
        # a one-token decode step, values growing now and then: older slots of
        # the partly filled blocks get re-encoded
        lens = [min(n + 1, f) for n, f in zip(lens, final)]
        step(lens, 1, 1.0 + (s % 7 == 3) * 4.0 + s * 0.1)
    say(f"  D={D} 30 decode steps ok")


def test_append_fp8_zero_values_and_short_sequences(api):
    g = torch.Generator().manual_seed(5)
    H, D, nb = 2, 128, 8
    tables = torch.tensor([[3, 5], [1, -1]], dtype=torch.int32)
    sl = torch.tensor([2, 20], dtype=torch.int32)
    kc, ks = _stale(g, nb, H, D)
    kn = torch.zeros(2, H, 6, D, dtype=torch.bfloat16)
    vn = torch.randn(2, H, 6, D, generator=g).to(torch.bfloat16)
    dk, dks, dv, dvs = kc.cuda(), ks.cuda(), kc.clone().cuda(), ks.clone().cuda()
    api.attn_paged_append_fp8(kn.cuda(), vn.cuda(), dk, dv, dks, dvs, tables.cuda(), sl.cuda())
    ref = oracle.quantize_append(kc, ks, kc, ks, tables, sl, kn, vn)
    torch.cuda.synchronize()
    assert _same(dk, ref[0]) and _same(dks, ref[1]) and _same(dv, ref[2]) and _same(dvs, ref[3])


def test_copy_blocks_fp8_bit_exact(api):
    g = torch.Generator().manual_seed(6)
    H, D, nb = 40, 128, 12
    kc, ks = _stale(g, nb, H, D)
    vc, vs = _stale(g, nb, H, D)
    src = torch.tensor([4, 9, 0], dtype=torch.int32)
    dst = torch.tensor([1, 11, 7], dtype=torch.int32)
    dk, dv, dks, dvs = kc.cuda(), vc.cuda(), ks.cuda(), vs.cuda()
    api.attn_paged_copy_blocks_fp8(dk, dv, dks, dvs, src.cuda(), dst.cuda())
    rk, rv = oracle.copy_blocks(kc, vc, src, dst)
    rks, rvs = oracle.copy_blocks(ks, vs, src, dst)
    torch.cuda.synchronize()
    assert torch.equal(dk.cpu(), rk) and torch.equal(dv.cpu(), rv)
    assert torch.equal(dks.cpu(), rks) and torch.equal(dvs.cpu(), rvs)


def _run(api, inp, splits=0, causal=True, scale=None):
    D = inp.q.shape[3]
    scale = scale if scale is not None else 1.0 / math.sqrt(D)
    o, lse = api.attn_paged_decode_fp8(inp.q.cuda(), inp.k_codes.cuda(), inp.v_codes.cuda(),
                                       inp.k_scale.cuda(), inp.v_scale.cuda(),
                                       inp.block_tables.cuda(), inp.seq_lens.cuda(),
                                       causal=causal, scale=scale, num_splits=splits,
                                       return_lse=True)
    torch.cuda.synchronize()
    return o, lse


def _ref(inp, causal=True, scale=None, heads=None):
    D = inp.q.shape[3]
    scale = scale if scale is not None else 1.0 / math.sqrt(D)
    return oracle.paged_attention_fp8(inp.q, inp.k_codes, inp.k_scale, inp.v_codes, inp.v_scale,
                                      inp.block_tables, inp.seq_lens, scale, causal, heads=heads)


def _err(o, lse, ref_o, ref_lse, pairs=None):
    g = o.double().cpu().numpy()
    gl = lse.double().cpu().numpy()
    if pairs is None:
        return float(np.abs(g - ref_o).max()), float(np.abs(gl - ref_lse).max())
    e = max(float(np.abs(g[b, h] - ref_o[b, h]).max()) for b, h in pairs)
    el = max(float(np.abs(gl[b, h] - ref_lse[b, h]).max()) for b, h in pairs)
    return e, el


FP8_CASES = [
    # (B, H, q_len, D, len range, q_heads, splits)
    (4, 3, 1, 128, (1, 300), 0, 0),
    (3, 2, 5, 128, (40, 1100), 0, 3),
    (5, 2, 1, 64, (17, 700), 0, 0),
    (4, 2, 1, 128, (100, 2000), 16, 0),   # grouped-query, group 8
    (2, 2, 4, 128, (300, 900), 8, 16),    # group 4 x q_len 4
]


@pytest.mark.parametrize("B,H,q_len,D,lens,qh,splits", FP8_CASES)
def test_decode_fp8(api, B, H, q_len, D, lens, qh, splits):
    spec = PagedSpec("fp8", B, H, q_len, D, seed=50 + B + H + q_len + D, len_lo=lens[0],
                     len_hi=lens[1], extra_blocks=3, poison=True, q_heads=qh)
    inp = paged_inputs_fp8(spec)
    say(f"fp8 decode B={B} H={H} q_len={q_len} D={D} lens={inp.seq_lens.tolist()} qh={qh} S={splits}")
    o, lse = _run(api, inp, splits)
    ro, rl = _ref(inp)
    e, el = _err(o, lse, ro, rl)
    say(f"  max|dO|={e:.3e} max|dlse|={el:.3e}")
    assert torch.isfinite(o.float()).all()
    assert e <= TOL_BF16 and el <= TOL_LSE


@pytest.mark.parametrize("splits", [0, 1])
def test_decode_fp8_pool_past_2pow31_bytes_matches_compact_pool(api, splits):
    """FP8 code pools of 131200 blocks of 8 heads x 16 x 128 hold more than 2^31
    bytes each; blocks from 131072 on start past byte 2^31. The problem's blocks
    moved to the end of such pools (every other block NaN codes and NaN
    scales) give bit-identical outputs and log-sum-exps to the compact pools."""
    spec = PagedSpec("fp8_big_pool", 3, 8, 1, 128, seed=77, len_lo=200, len_hi=1200, extra_blocks=3,
                     poison=True)
    inp = paged_inputs_fp8(spec)
    nb_big = 131200
    assert nb_big * 8 * 16 * 128 > 2**31 and 131072 * 8 * 16 * 128 == 2**31
    n_small = inp.k_codes.shape[0]
    off = nb_big - n_small
    tab = inp.block_tables.clone()
    tab[tab >= 0] += off
    used = tab[tab >= 0]
    assert int(used.max()) < nb_big and int((used >= 131072).sum()) > 0
    dev = torch.device("cuda")
    k_big = torch.full((nb_big, 8, BS, 128), 0x7F, dtype=torch.uint8, device=dev)
    v_big = torch.full_like(k_big, 0x7F)
    ks_big = torch.full((nb_big, 8), float("nan"), dtype=torch.float32, device=dev)
    vs_big = torch.full_like(ks_big, float("nan"))
    k_big[off:] = inp.k_codes.to(dev)
    v_big[off:] = inp.v_codes.to(dev)
    ks_big[off:] = inp.k_scale.to(dev)
    vs_big[off:] = inp.v_scale.to(dev)
    say(f"fp8 decode, pools of {nb_big} blocks, lens={inp.seq_lens.tolist()} S={splits}")
    o1, l1 = _run(api, inp, splits)
    o2, l2 = api.attn_paged_decode_fp8(inp.q.cuda(), k_big, v_big, ks_big, vs_big, tab.cuda(),
                                       inp.seq_lens.cuda(), causal=True, scale=1.0 / math.sqrt(128),
                                       num_splits=splits, return_lse=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o1.float()).all()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    e, el = _err(o2, l2, *_ref(inp))
    say(f"  max|dO|={e:.3e} max|dlse|={el:.3e}")
    assert e <= TOL_BF16 and el <= TOL_LSE
    del k_big, v_big, ks_big, vs_big
    torch.cuda.empty_cache()


@pytest.mark.parametrize("scale", [0.0, -0.05, 0.3])
def test_decode_fp8_other_scales_and_full_attention(api, scale):
    spec = PagedSpec("fp8s", 3, 2, 3, 128, seed=61, len_lo=20, len_hi=400, poison=True)
    inp = paged_inputs_fp8(spec)
    for causal in (True, False):
        o, lse = _run(api, inp, 2, causal, scale)
        ro, rl = _ref(inp, causal, scale)
        e, el = _err(o, lse, ro, rl)
        assert e <= TOL_BF16 and el <= TOL_LSE, (causal, e, el)


def test_decode_fp8_of_appended_tokens(api):
    """Tokens quantised by the append kernel are read back by the decode kernel:
    the oracle gets the same bf16 tokens and runs its own quantiser."""
    g = torch.Generator().manual_seed(62)
    H, D, nb, width = 4, 128, 40, 10
    lens = [150, 33, 97]
    tables = _tables(g, lens, nb, width)
    kc = torch.zeros((nb, H, BS, D), dtype=torch.uint8)
    ks = torch.zeros((nb, H))
    kn = torch.randn(3, H, max(lens), D, generator=g).to(torch.bfloat16)
    vn = torch.randn(3, H, max(lens), D, generator=g).to(torch.bfloat16)
    sl = torch.tensor(lens, dtype=torch.int32)
    dk, dv, dks, dvs = kc.cuda(), kc.clone().cuda(), ks.cuda(), ks.clone().cuda()
    api.attn_paged_append_fp8(kn.cuda(), vn.cuda(), dk, dv, dks, dvs, tables.cuda(), sl.cuda())
    ref = oracle.quantize_append(kc, ks, kc, ks, tables, sl, kn, vn)
    q = torch.randn(3, H, 1, D, generator=g).to(torch.bfloat16)
    o, lse = api.attn_paged_decode_fp8(q.cuda(), dk, dv, dks, dvs, tables.cuda(), sl.cuda(),
                                       return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.paged_attention_fp8(q, ref[0], ref[1], ref[2], ref[3], tables, sl,
                                        1 / math.sqrt(D), True)
    e, el = _err(o, lse, ro, rl)
    say(f"  appended fp8 decode max|dO|={e:.3e}")
    assert e <= TOL_BF16 and el <= TOL_LSE
    # and the quantised cache stays close to the bf16 tokens: attention over
    # the bf16 values differs by the quantisation error only
    rb, _ = oracle.dense_attention(q[0, 0], kn[0, 0, -lens[0]:], vn[0, 0, -lens[0]:],
                                   1 / math.sqrt(D), True)
    assert np.abs(ro[0, 0] - rb).max() < 0.1


def test_decode_fp8_full_size(api):
    inp = paged_inputs_fp8(C4F8)
    o, lse = _run(api, inp, C4F8.num_splits)
    ro, rl = _ref(inp)
    e, el = _err(o, lse, ro, rl)
    say(f"  fp8 decode full size, all pairs: max|dO|={e:.3e} max|dlse|={el:.3e}")
    assert torch.isfinite(o.float()).all()
    assert e <= TOL_BF16 and el <= TOL_LSE
