"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module draws random numbers and lays them out; it holds none of the
attention arithmetic, so both the HIP path and the CPU oracle may use it.

Recipe (every draw comes from one ``torch.Generator`` seeded per workload, on
the CPU, in the order listed, so the same seed gives the same bytes anywhere):

* prefill: Q, K, V ~ N(0, 1) drawn as float32 in that order, each [B, H, L, D];
  cast to bfloat16 (round to nearest even) for bf16 workloads.
* paged: seq_lens (uniform integers, or fixed), then a random permutation of
  the physical block ids, then K pool, V pool, then q, all N(0, 1) float32 cast
  to bfloat16. Sequence b takes the next ceil(seq_len_b / 16) ids of the
  permutation as its block table (an optional shared prefix of ids comes first
  in every row); unused table entries are -1. Pools are [num_blocks, H, 16, D].
  Tail slots past seq_len hold random values too (or NaN when ``poison``), and
  ``extra_blocks`` adds pool blocks that no table references.
* FP8 paged (E4M3 codes with per-(block, head) float32 scales): the same
  layout draws, then K codes, V codes, K scales, V scales, q. A code is a
  uniform sign bit over a uniform magnitude code in [0x30, 0x70] (values
  0.5 .. 128 before scaling); scales are uniform in [1e-3, 4e-3]. With
  ``poison`` every slot no sequence may read holds the NaN code 0x7F.
"""

import math
from dataclasses import dataclass, field

import torch

BLOCK = 16


@dataclass(frozen=True)
class PrefillSpec:
    name: str
    B: int
    H: int
    L: int
    D: int
    dtype: str  # "f32" or "bf16"
    causal: bool
    seed: int

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.D)


@dataclass(frozen=True)
class PagedSpec:
    name: str
    B: int
    H: int
    q_len: int
    D: int
    seed: int
    len_lo: int = 0          # seq_lens ~ U[len_lo, len_hi] when fixed_len is 0
    len_hi: int = 0
    fixed_len: int = 0
    shared_prefix_blocks: int = 0
    num_splits: int = 0      # 0 = library's choice
    max_blocks_per_seq: int = 0  # 0 = ceil(max possible length / 16)
    causal: bool = True
    extra_blocks: int = 0
    poison: bool = False
    q_heads: int = 0         # query heads when the pools hold fewer (grouped-query); 0 = H

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.D)

    @property
    def table_width(self):
        if self.max_blocks_per_seq:
            return self.max_blocks_per_seq
        top = self.fixed_len if self.fixed_len else self.len_hi
        return -(-top // BLOCK)


# The five workloads the library is measured on.
C1 = PrefillSpec("c1_prefill_f32_1x1x128x64_causal", 1, 1, 128, 64, "f32", True, 1)
C2 = PrefillSpec("c2_prefill_bf16_8x16x1024x128_causal", 8, 16, 1024, 128, "bf16", True, 2)
C3 = PrefillSpec("c3_prefill_bf16_1x40x4096x128_causal", 1, 40, 4096, 128, "bf16", True, 3)
C4 = PagedSpec("c4_paged_decode_bf16_64seq_40h_len128-4096", 64, 40, 1, 128, 4,
               len_lo=128, len_hi=4096)
C5 = PagedSpec("c5_paged_verify_bf16_4seq_40h_q5_len32768_prefix2048_s16", 4, 40, 5, 128, 5,
               fixed_len=32768, shared_prefix_blocks=128, num_splits=16)
# Grouped-query decode (a follow-on of the paged path): 64 query heads reading 8
# KV heads (group 8), the c4 length mix.
C4G = PagedSpec("gqa_paged_decode_bf16_64seq_64qh_8kvh_len128-4096", 64, 8, 1, 128, 6,
                len_lo=128, len_hi=4096, q_heads=64)
# Chunked prefill over the paged cache (a follow-on of the paged path): 8
# sequences x 40 heads, a 512-token chunk after a 3584-token cached prefix.
CPF = PagedSpec("chunked_prefill_bf16_8seq_40h_chunk512_len4096", 8, 40, 512, 128, 7,
                fixed_len=4096)
# FP8 cache (a follow-on of the paged path): the c4 decode workload with E4M3
# K/V codes and per-(block, head) scales.
C4F8 = PagedSpec("fp8_paged_decode_64seq_40h_len128-4096", 64, 40, 1, 128, 8,
                 len_lo=128, len_hi=4096)
CONFIGS = {"c1": C1, "c2": C2, "c3": C3, "c4": C4, "c5": C5, "c4g": C4G, "cpf": CPF,
           "c4f8": C4F8}


def _randn(gen, shape, dtype):
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    return x.to(torch.bfloat16) if dtype == "bf16" else x


def prefill_inputs(spec):
    """(q, k, v) CPU tensors [B, H, L, D] for a PrefillSpec."""
    g = torch.Generator().manual_seed(spec.seed)
    shape = (spec.B, spec.H, spec.L, spec.D)
    q = _randn(g, shape, spec.dtype)
    k = _randn(g, shape, spec.dtype)
    v = _randn(g, shape, spec.dtype)
    return q, k, v


@dataclass
class PagedInputs:
    q: torch.Tensor            # [B, H, q_len, D] bf16
    k_pool: torch.Tensor       # [num_blocks, H, 16, D] bf16
    v_pool: torch.Tensor
    block_tables: torch.Tensor  # [B, width] int32, -1 padded
    seq_lens: torch.Tensor     # [B] int32
    perm: torch.Tensor = field(repr=False, default=None)


def paged_layout(spec, gen=None):
    """seq_lens, block_tables and num_blocks for a PagedSpec (no pools)."""
    g = gen if gen is not None else torch.Generator().manual_seed(spec.seed)
    if spec.fixed_len:
        lens = torch.full((spec.B,), spec.fixed_len, dtype=torch.int64)
    else:
        lens = torch.randint(spec.len_lo, spec.len_hi + 1, (spec.B,), generator=g, dtype=torch.int64)
    nb = [(-(-int(n) // BLOCK)) for n in lens]
    sp = spec.shared_prefix_blocks
    own = [max(n - sp, 0) for n in nb]
    used = sp + sum(own)
    total = used + spec.extra_blocks
    perm = torch.randperm(total, generator=g, dtype=torch.int64)
    width = max(spec.table_width, max(nb) if nb else 0)
    tables = torch.full((spec.B, width), -1, dtype=torch.int64)
    shared = perm[:sp]
    pos = sp
    for b in range(spec.B):
        row = torch.cat([shared[:min(sp, nb[b])], perm[pos:pos + own[b]]])
        pos += own[b]
        tables[b, :row.numel()] = row
    return lens.to(torch.int32), tables.to(torch.int32), total, perm


def paged_inputs(spec):
    """Full PagedInputs on the CPU for a PagedSpec."""
    g = torch.Generator().manual_seed(spec.seed)
    lens, tables, total, perm = paged_layout(spec, g)
    shape = (total, spec.H, BLOCK, spec.D)
    k_pool = _randn(g, shape, "bf16")
    v_pool = _randn(g, shape, "bf16")
    q = _randn(g, (spec.B, spec.q_heads or spec.H, spec.q_len, spec.D), "bf16")
    if spec.poison:
        _poison(k_pool, v_pool, lens, tables)
    return PagedInputs(q, k_pool, v_pool, tables, lens, perm)


@dataclass
class PagedInputsFp8:
    q: torch.Tensor            # [B, Hq, q_len, D] bf16
    k_codes: torch.Tensor      # [num_blocks, H, 16, D] uint8 E4M3 codes
    v_codes: torch.Tensor
    k_scale: torch.Tensor      # [num_blocks, H] float32
    v_scale: torch.Tensor
    block_tables: torch.Tensor
    seq_lens: torch.Tensor


def paged_inputs_fp8(spec):
    """FP8 paged inputs on the CPU for a PagedSpec (recipe in the module docstring)."""
    g = torch.Generator().manual_seed(spec.seed)
    lens, tables, total, _ = paged_layout(spec, g)
    shape = (total, spec.H, BLOCK, spec.D)

    def codes():
        mag = torch.randint(0x30, 0x71, shape, generator=g, dtype=torch.uint8)
        sign = torch.randint(0, 2, shape, generator=g, dtype=torch.uint8) * 0x80
        return mag | sign

    k, v = codes(), codes()
    ks = torch.rand((total, spec.H), generator=g) * 3e-3 + 1e-3
    vs = torch.rand((total, spec.H), generator=g) * 3e-3 + 1e-3
    q = _randn(g, (spec.B, spec.q_heads or spec.H, spec.q_len, spec.D), "bf16")
    if spec.poison:
        readable = torch.zeros(total, BLOCK, dtype=torch.bool)
        for b in range(tables.shape[0]):
            n = int(lens[b])
            for t0 in range(0, n, BLOCK):
                readable[int(tables[b, t0 // BLOCK]), : min(BLOCK, n - t0)] = True
        idx = (~readable).nonzero(as_tuple=True)
        k[idx[0], :, idx[1], :] = 0x7F
        v[idx[0], :, idx[1], :] = 0x7F
    return PagedInputsFp8(q, k, v, ks, vs, tables, lens)


def _poison(k_pool, v_pool, lens, tables):
    """NaN in every pool slot that no sequence may read."""
    readable = torch.zeros(k_pool.shape[0], BLOCK, dtype=torch.bool)
    for b in range(tables.shape[0]):
        n = int(lens[b])
        for t0 in range(0, n, BLOCK):
            readable[int(tables[b, t0 // BLOCK]), : min(BLOCK, n - t0)] = True
    mask = ~readable
    k_pool[mask.nonzero(as_tuple=True)[0], :, mask.nonzero(as_tuple=True)[1], :] = float("nan")
    v_pool[mask.nonzero(as_tuple=True)[0], :, mask.nonzero(as_tuple=True)[1], :] = float("nan")


def permute_pool(inp, seed):
    """Same logical cache under a different physical placement of its blocks.

    Block i of the pool moves to position sigma[i]; tables are remapped so
    every sequence still reads the same rows.
    """
    g = torch.Generator().manual_seed(seed)
    n = inp.k_pool.shape[0]
    sigma = torch.randperm(n, generator=g)
    k2 = torch.empty_like(inp.k_pool)
    v2 = torch.empty_like(inp.v_pool)
    k2[sigma] = inp.k_pool
    v2[sigma] = inp.v_pool
    t = inp.block_tables.to(torch.int64)
    t2 = torch.where(t >= 0, sigma[t.clamp(min=0)], t).to(torch.int32)
    return PagedInputs(inp.q, k2, v2, t2, inp.seq_lens, None)
