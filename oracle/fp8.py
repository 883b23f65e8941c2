"""FP8 (E4M3) KV cache with block-wise scales: encoding, appends, attention.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The FlashAttention-3 item of [P3] lists FP8 data (E4M3 / E5M2) for the
attention products, with block-wise quantisation: every block carries its own
scale factor, which keeps FP8's narrow range usable. The deployment example of
[P2] §五 runs a server with an FP8 KV cache. Here the cache blocks of the
paged pool ([P1] §3.2) are those blocks: each (physical block, head) of K and
of V holds 16 x D E4M3 codes and one float32 scale, and a stored value means
decode(code) * scale.

Readings taken where the pages leave the steps open (listed in the design
notes with their reasons):
  * E4M3 is the OCP 8-bit format: 1 sign, 4 exponent (bias 7), 3 mantissa
    bits; exponent 0 is subnormal (2^-6 * m / 8); codes 0x7F / 0xFF are NaN;
    the largest finite magnitude is 448.
  * encoding rounds to the nearest representable value, ties to the even code
    (mantissa LSB 0), after clamping to [-448, 448]; a negative value that
    rounds to zero keeps its sign (code 0x80).
  * scale of a (block, head): it only grows. An append computes
    s_new = max(s_old, amax(new values) / 448), where s_old is the stored scale,
    or 0 when the append starts at slot 0 of the block (the block starts
    afresh). If s_new > s_old the slots already in the block are re-encoded as
    encode((decode(code) * s_old) / s_new). New values are encoded as
    encode(x / s_new); with s_new = 0 (all new values zero) codes are 0.
  * the arithmetic that decides codes (amax / 448, the products and
    quotients) is float32 with round-to-nearest-even, the precision the
    kernels use, so both sides reach the same integers.
  * slots past the last written position keep whatever they held; nothing
    reads them.
"""

import numpy as np

try:
    import torch
except ImportError:  # pragma: no cover
    torch = None

from .attention import dense_attention, paged_gather

E4M3_MAX = 448.0


def _np(x):
    if torch is not None and isinstance(x, torch.Tensor):
        return x.detach().cpu().numpy()
    return np.asarray(x)


def _f32(x):
    if torch is not None and isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float32).numpy()
    return np.asarray(x, dtype=np.float32)


def _decode_one(c):
    sign = -1.0 if c & 0x80 else 1.0
    e = (c >> 3) & 15
    m = c & 7
    if e == 15 and m == 7:
        return np.nan
    if e == 0:
        return sign * 2.0 ** -6 * (m / 8.0)
    return sign * 2.0 ** (e - 7) * (1.0 + m / 8.0)


DECODE_TABLE = np.array([_decode_one(c) for c in range(256)])  # float64, exact


def e4m3_decode(codes):
    """Exact value (float64) of each E4M3 code."""
    return DECODE_TABLE[_np(codes).astype(np.int64)]


# non-negative finite values and their codes, ascending (0x00 .. 0x7E)
_POS_CODES = np.arange(0, 0x7F)
_POS_VALS = DECODE_TABLE[_POS_CODES]


def e4m3_encode(x):
    """E4M3 code of float32 values: clamp to +-448, round to nearest, ties even."""
    x = np.asarray(x, dtype=np.float32)
    a = np.minimum(np.abs(x.astype(np.float64)), E4M3_MAX)
    hi = np.searchsorted(_POS_VALS, a, side="left")        # first value >= a
    hi = np.minimum(hi, len(_POS_VALS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALS[lo]
    d_hi = _POS_VALS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    mag = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    return (mag | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def quantize_append(k_codes, k_scale, v_codes, v_scale, block_tables, seq_lens, k_new, v_new,
                    block_size=16):
    """Write new tokens into an FP8 paged cache; returns the updated copies.

    k_codes, v_codes [num_blocks, H, block_size, D] uint8; k_scale, v_scale
    [num_blocks, H] float32; k_new, v_new [B, H, n_new, D] (any float dtype,
    finite). Token t of sequence b sits at position seq_lens[b] - n_new + t
    (seq_lens count the new tokens); negative positions, and blocks whose
    table entry is negative, are skipped. Each
    (block, head) that receives tokens follows the scale rule of the module
    docstring.
    """
    tables = _np(block_tables).astype(np.int64)
    lens = _np(seq_lens).astype(np.int64)
    out = []
    for codes, scale, new in ((k_codes, k_scale, k_new), (v_codes, v_scale, v_new)):
        c = np.array(_np(codes), dtype=np.uint8, copy=True)
        s = np.array(_f32(scale), dtype=np.float32, copy=True)
        x = _f32(new)
        n_new = x.shape[2]
        H = c.shape[1]
        for b in range(tables.shape[0]):
            first = max(int(lens[b]) - n_new, 0)
            last = int(lens[b])  # exclusive
            p = first
            while p < last:
                lb = p // block_size
                s0 = p - lb * block_size
                s1 = min(last - lb * block_size, block_size)
                phys = int(tables[b][lb])
                t0 = lb * block_size + s0 - (int(lens[b]) - n_new)
                p = lb * block_size + s1
                if phys < 0:  # no block assigned: nothing is placed
                    continue
                for h in range(H):
                    vals = x[b, h, t0:t0 + (s1 - s0)]                     # [n, D] float32
                    amax = np.float32(np.max(np.abs(vals))) if vals.size else np.float32(0)
                    s_old = np.float32(0) if s0 == 0 else s[phys, h]
                    s_new = max(s_old, np.float32(amax / np.float32(E4M3_MAX)))
                    if s_new > s_old and s0 > 0:
                        old = e4m3_decode(c[phys, h, :s0]).astype(np.float32)
                        c[phys, h, :s0] = e4m3_encode((old * s_old) / s_new)
                    if s_new > 0:
                        c[phys, h, s0:s1] = e4m3_encode(vals / s_new)
                    else:
                        c[phys, h, s0:s1] = 0
                    s[phys, h] = s_new
        out += [c, s]
    return tuple(out)


def dequantize(codes, scales):
    """decode(code) * scale in float64: [N, H, bs, D] codes, [N, H] scales."""
    return e4m3_decode(codes) * _f32(scales).astype(np.float64)[:, :, None, None]


def paged_attention_fp8(q, k_codes, k_scale, v_codes, v_scale, block_tables, seq_lens, scale,
                        causal, block_size=16, heads=None):
    """paged_attention over an FP8 cache: keys and values are the dequantised
    stored values decode(code) * scale of their (block, head). Grouped-query
    heads as in paged_attention. Returns (o, lse) in float64."""
    B, Hq, lq, D = q.shape
    hkv = _np(k_codes).shape[1]
    if Hq % hkv != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    group = Hq // hkv
    o = np.full((B, Hq, lq, D), np.nan)
    lse = np.full((B, Hq, lq), np.nan)
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    tables = _np(block_tables).astype(np.int64)
    lens = _np(seq_lens).astype(np.int64)
    kc_all, vc_all = _np(k_codes), _np(v_codes)
    ks_all, vs_all = _f32(k_scale), _f32(v_scale)
    for b in sorted({b for b, _ in pairs}):
        n = int(lens[b])
        tok = np.arange(n)
        phys = tables[b][tok // block_size]
        kc = paged_gather(kc_all, tables[b:b + 1], lens[b:b + 1], block_size)[0]  # [H, n, D]
        vc = paged_gather(vc_all, tables[b:b + 1], lens[b:b + 1], block_size)[0]
        kd = e4m3_decode(kc) * ks_all[phys].T.astype(np.float64)[:, :, None]
        vd = e4m3_decode(vc) * vs_all[phys].T.astype(np.float64)[:, :, None]
        for bb, h in pairs:
            if bb == b:
                o[b, h], lse[b, h] = dense_attention(q[b, h], kd[h // group], vd[h // group],
                                                     scale, causal)
    return o, lse
