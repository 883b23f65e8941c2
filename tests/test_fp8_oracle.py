"""Pins of the FP8 (E4M3) cache oracle.

* decode / encode against torch's float8_e4m3fn (a library implementation of
  the same OCP format), on every code and on values that sit exactly between
  neighbours (ties), plus the format's fixed points (448, smallest subnormal);
* the append rule against properties that do not re-run it: error bounds,
  the block maximum landing on +-448, exactness on representable inputs,
  chunking invariance while the scale stands still, exact re-encoding when the
  scale grows by a power of two, and a fresh block ignoring a stale scale;
* attention over the FP8 cache against scalar loops on values dequantised
  through torch's decoder.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.test_oracle_pins import brute_attention

BS = 16


def torch_decode(codes):
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8).copy())
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_encode(x):
    t = torch.from_numpy(np.asarray(x, dtype=np.float32).copy())
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_matches_library_on_every_code():
    codes = np.arange(256)
    ours = oracle.e4m3_decode(codes)
    ref = torch_decode(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and np.isnan(ours[0x7F])
    assert ours[0x08] == 2.0 ** -6  # smallest normal


def test_encode_matches_library_on_values_and_ties():
    fin = oracle.e4m3_decode(np.arange(0x7F))
    mids = (fin[1:] + fin[:-1]) / 2                  # exact ties
    rng = np.random.default_rng(0)
    x = np.concatenate([fin, -fin, mids, -mids,
                        np.nextafter(mids.astype(np.float32), np.float32(1e9)),
                        np.nextafter(mids.astype(np.float32), np.float32(-1e9)),
                        rng.uniform(-448, 448, 20000), rng.standard_normal(5000) * 1e-3])
    x = x.astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(x), torch_encode(x))


def test_encode_clamps_out_of_range():
    assert oracle.e4m3_encode(np.float32([1e6, -500.0, 449.0])).tolist() == [0x7E, 0xFE, 0x7E]


def _cache(nb, H, D, seed=0):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 0x7E, (nb, H, BS, D)).astype(np.uint8)   # stale contents
    scales = rng.uniform(0.5, 2.0, (nb, H)).astype(np.float32)
    return codes, scales


def test_append_fresh_blocks_error_bound_and_max_code():
    rng = np.random.default_rng(1)
    H, D = 2, 8
    kc, ks = _cache(4, H, D)
    vc, vs = _cache(4, H, D, 1)
    x = (rng.standard_normal((1, H, 40, D)) * 3).astype(np.float32)
    table = np.array([[2, 0, 3]])
    kc2, ks2, vc2, vs2 = oracle.quantize_append(kc, ks, vc, vs, table, [40], x, -x)
    deq = oracle.dequantize(kc2, ks2)
    for lb, phys in enumerate([2, 0, 3]):
        n = min(40 - lb * BS, BS)
        for h in range(H):
            blk = x[0, h, lb * BS: lb * BS + n]
            amax = np.abs(blk).max()
            s = ks2[phys, h]
            assert s == np.float32(np.float32(amax) / np.float32(448))
            got = deq[phys, h, :n]
            # relative error 2^-4 in the normal range, s * 2^-10 below it
            bound = np.maximum(np.abs(blk) * 2.0 ** -4, float(s) * 2.0 ** -10)
            assert np.all(np.abs(got - blk) <= bound + 1e-12)
            arg = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
            assert kc2[phys, h, arg[0], arg[1]] & 0x7F == 0x7E
            # V got the negated values: same scale, mirrored codes
            assert vs2[phys, h] == s and np.array_equal(vc2[phys, h, :n], kc2[phys, h, :n] ^ 0x80)
    # the untouched block 1 and the slots past position 40 are unchanged
    assert np.array_equal(kc2[1], kc[1]) and ks2[1].tolist() == ks[1].tolist()
    assert np.array_equal(kc2[3, :, 8:], kc[3, :, 8:])


def test_append_exact_on_representable_values():
    """Values decode(code) * 2^k with the block max at 448 * 2^k come back exactly."""
    rng = np.random.default_rng(2)
    H, D = 1, 16
    codes = rng.integers(0, 0x7E, (1, H, BS, D))
    codes[0, 0, 3, 5] = 0x7E
    x = (oracle.e4m3_decode(codes) * 2.0 ** -3).astype(np.float32)
    kc, ks = _cache(1, H, D)
    kc2, ks2, _, _ = oracle.quantize_append(kc, ks, kc, ks, [[0]], [BS], x, x)
    assert ks2[0, 0] == 2.0 ** -3
    assert np.array_equal(oracle.dequantize(kc2, ks2)[0], x.astype(np.float64)[0])


def test_append_in_pieces_equals_at_once_while_scale_stands():
    rng = np.random.default_rng(3)
    H, D = 2, 8
    x = rng.standard_normal((2, H, 30, D)).astype(np.float32)
    x[:, :, 0, 0] = 10.0   # the first token holds each block's maximum
    x[:, :, 16, 0] = 10.0
    kc, ks = _cache(6, H, D)
    table = np.array([[0, 1, -1], [4, 5, -1]])
    lens = np.array([30, 30])
    one = oracle.quantize_append(kc, ks, kc, ks, table, lens, x, x)
    step = (kc, ks, kc, ks)
    for a, b in ((0, 1), (1, 7), (7, 16), (16, 17), (17, 30)):
        step = oracle.quantize_append(step[0], step[1], step[2], step[3], table, lens - (30 - b),
                                      x[:, :, a:b], x[:, :, a:b])
    for u, v in zip(one, step):
        assert np.array_equal(u, v)


def test_append_growing_scale_reencodes_old_slots():
    """A later token 4x larger: the scale grows 4x (a power of two), so the old
    codes are re-encoded exactly (exponent shift) unless they underflow."""
    H, D = 1, 4
    first = np.array([[[[0.5, -1.0, 0.25, 2.0]]]], dtype=np.float32)       # amax 2
    second = np.array([[[[8.0, 0.5, -0.5, 1.0]]]], dtype=np.float32)       # amax 8
    kc, ks = _cache(1, H, D)
    a = oracle.quantize_append(kc, ks, kc, ks, [[0]], [1], first, first)
    assert a[1][0, 0] == np.float32(2.0) / np.float32(448)
    b = oracle.quantize_append(a[0], a[1], a[2], a[3], [[0]], [2], second, second)
    assert b[1][0, 0] == np.float32(8.0) / np.float32(448)
    deq = oracle.dequantize(b[0], b[1])[0, 0]
    np.testing.assert_allclose(deq[0], first[0, 0, 0], rtol=2.0 ** -4)
    np.testing.assert_allclose(deq[1], second[0, 0, 0], rtol=2.0 ** -4)
    # the old token's codes move down two binades: exponent field - 2, same mantissa
    old = a[0][0, 0, 0].astype(int)
    new = b[0][0, 0, 0].astype(int)
    assert np.array_equal(new & 0x80, old & 0x80)
    assert np.array_equal(new & 0x7F, (old & 0x7F) - (2 << 3))
    assert b[0][0, 0, 0, 3] == 0x6E                # 2.0 at scale 8/448 is 112 = 1.75 * 2^6
    assert b[0][0, 0, 1, 0] == 0x7E


def test_append_at_slot_zero_ignores_a_stale_scale():
    kc, ks = _cache(2, 1, 4)
    ks[:] = 1e6                                   # stale, huge
    x = np.array([[[[1.0, 2.0, 3.0, 4.0]]]], dtype=np.float32)
    c2, s2, _, _ = oracle.quantize_append(kc, ks, kc, ks, [[1]], [1], x, x)
    assert s2[1, 0] == np.float32(4.0) / np.float32(448)
    np.testing.assert_allclose(oracle.dequantize(c2, s2)[1, 0, 0], x[0, 0, 0], rtol=2.0 ** -4)


def test_append_skips_unassigned_blocks():
    """A table entry of -1 places nothing (and must not wrap to the last block)."""
    kc, ks = _cache(3, 1, 4)
    x = np.ones((1, 1, 6, 4), dtype=np.float32)
    c2, s2, _, _ = oracle.quantize_append(kc, ks, kc, ks, [[1, -1]], [20], x, x)
    assert np.array_equal(c2[2], kc[2]) and s2[2, 0] == ks[2, 0]
    assert np.array_equal(c2[0], kc[0])
    # block 1 got slots 14, 15 over its stored scale, which already covers them
    assert s2[1, 0] == max(ks[1, 0], np.float32(1) / np.float32(448))
    assert np.array_equal(c2[1, 0, :14], kc[1, 0, :14])
    assert (c2[1, 0, 14:] == oracle.e4m3_encode(np.float32(1) / s2[1, 0])).all()


def test_append_all_zero_block_has_zero_scale():
    kc, ks = _cache(1, 1, 4)
    z = np.zeros((1, 1, 3, 4), dtype=np.float32)
    c2, s2, _, _ = oracle.quantize_append(kc, ks, kc, ks, [[0]], [3], z, z)
    assert s2[0, 0] == 0 and (c2[0, 0, :3] == 0).all()


def test_fp8_attention_against_scalar_loops():
    rng = np.random.default_rng(5)
    H, D, nb = 2, 8, 6
    kc = rng.integers(0, 0x7E, (nb, H, BS, D)).astype(np.uint8) | (rng.integers(0, 2, (nb, H, BS, D)) * 0x80).astype(np.uint8)
    vc = rng.integers(0, 0x7E, (nb, H, BS, D)).astype(np.uint8)
    ks = rng.uniform(1e-3, 1e-2, (nb, H)).astype(np.float32)
    vs = rng.uniform(1e-3, 1e-2, (nb, H)).astype(np.float32)
    table = np.array([[4, 1, 3], [0, 5, -1]])
    lens = np.array([40, 20])
    q = torch.randn(2, H, 3, D, generator=torch.Generator().manual_seed(0))
    o, lse = oracle.paged_attention_fp8(q, kc, ks, vc, vs, table, lens, 0.3, True)
    for b in range(2):
        n = int(lens[b])
        for h in range(H):
            kk = [[float(torch_decode(kc[table[b][t // BS], h, t % BS, d])) * float(ks[table[b][t // BS], h])
                   for d in range(D)] for t in range(n)]
            vv = [[float(torch_decode(vc[table[b][t // BS], h, t % BS, d])) * float(vs[table[b][t // BS], h])
                   for d in range(D)] for t in range(n)]
            ob, lb = brute_attention(q[b, h].double().tolist(), kk, vv, 0.3, True)
            np.testing.assert_allclose(o[b, h], ob, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[b, h], lb, rtol=0, atol=1e-12)
