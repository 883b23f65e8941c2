"""CPU checks of the C ABI: the library loads, exports what include/attn.h
declares, and rejects bad arguments on the host before touching a device.

No call here reaches a kernel launch: each one fails validation first (the
pointers passed are fake but never dereferenced), so these run without a GPU.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


@pytest.fixture(scope="module")
def api():
    import attention_tiled_qk_amd as m
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(attn_[a-z_0-9]+)\s*\(", text, flags=re.M)))


def header_constants():
    text = open(HEADER).read()
    return {k: int(v) for k, v in re.findall(r"(ATTN_[A-Z_0-9]+)\s*=\s*(-?\d+)", text)}


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["attn_prefill", "attn_paged_decode", "attn_lse_merge", "attn_paged_gather",
              "attn_paged_workspace_bytes", "attn_status_string", "attn_version"]:
        assert n in names


def test_every_declared_symbol_is_exported(api):
    for name in declared_functions():
        assert hasattr(api.lib, name), name


def test_version(api):
    assert api.attn_version() == 100


FAKE = ctypes.c_void_p(1 << 20)       # 16-byte aligned, never dereferenced
FAKE_ODD = ctypes.c_void_p((1 << 20) + 4)


def test_status_strings(api):
    c = header_constants()
    for name, val in c.items():
        if name.startswith("ATTN_ERR_") or name == "ATTN_OK":
            s = api.lib.attn_status_string(val).decode()
            assert s and s != "unknown status"
    assert api.lib.attn_status_string(12345).decode() == "unknown status"


def test_prefill_rejects_bad_arguments(api):
    c = header_constants()
    L = api.lib
    ok = dict(B=1, H=1, Lq=128, D=64, causal=1, scale=0.125, dtype=0)

    def call(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, **kw):
        a = dict(ok, **kw)
        return L.attn_prefill(q, k, v, o, lse, a["B"], a["H"], a["Lq"], a["D"], a["causal"],
                              a["scale"], a["dtype"], None)

    assert call(q=None) == c["ATTN_ERR_NULL_PTR"]
    assert call(o=None) == c["ATTN_ERR_NULL_PTR"]
    assert call(B=0) == c["ATTN_ERR_BAD_SHAPE"]
    assert call(Lq=-3) == c["ATTN_ERR_BAD_SHAPE"]
    assert call(D=96) == c["ATTN_ERR_UNSUPPORTED"]
    assert call(D=256) == c["ATTN_ERR_UNSUPPORTED"]
    assert call(dtype=7) == c["ATTN_ERR_BAD_DTYPE"]
    assert call(causal=2) == c["ATTN_ERR_BAD_SHAPE"]
    assert call(scale=float("nan")) == c["ATTN_ERR_BAD_SHAPE"]
    assert call(scale=float("inf")) == c["ATTN_ERR_BAD_SHAPE"]
    assert call(k=FAKE_ODD) == c["ATTN_ERR_MISALIGNED"]
    assert call(B=1 << 20, H=1 << 20, Lq=1 << 20, D=128) == c["ATTN_ERR_OVERFLOW"]


def test_paged_decode_rejects_bad_arguments(api):
    c = header_constants()
    L = api.lib
    base = dict(B=2, H=4, q_len=1, D=128, nblk=10, width=8, bs=16, causal=1, scale=0.1,
                splits=1, ws=None, ws_bytes=0, dtype=1)

    def call(q=FAKE, kp=FAKE, vp=FAKE, bt=FAKE, sl=FAKE, o=FAKE, lse=None, **kw):
        a = dict(base, **kw)
        return L.attn_paged_decode(q, kp, vp, bt, sl, o, lse, a["B"], a["H"], a["q_len"], a["D"],
                                   a["nblk"], a["width"], a["bs"], a["causal"], a["scale"],
                                   a["splits"], a["ws"], a["ws_bytes"], a["dtype"], None)

    assert call(bt=None) == c["ATTN_ERR_NULL_PTR"]
    assert call(sl=None) == c["ATTN_ERR_NULL_PTR"]
    assert call(B=0) == c["ATTN_ERR_BAD_SHAPE"]
    assert call(nblk=0) == c["ATTN_ERR_BAD_SHAPE"]
    assert call(dtype=0) == c["ATTN_ERR_BAD_DTYPE"]
    assert call(bs=32) == c["ATTN_ERR_UNSUPPORTED"]
    assert call(q_len=17) == c["ATTN_ERR_UNSUPPORTED"]
    assert call(q_len=0) == c["ATTN_ERR_BAD_SHAPE"]
    assert call(D=80) == c["ATTN_ERR_UNSUPPORTED"]
    assert call(splits=65) == c["ATTN_ERR_UNSUPPORTED"]
    assert call(splits=-1) == c["ATTN_ERR_UNSUPPORTED"]
    assert call(o=FAKE_ODD) == c["ATTN_ERR_MISALIGNED"]
    assert call(H=70000) == c["ATTN_ERR_OVERFLOW"]
    # a split count above one needs a workspace of the advertised size
    need = L.attn_paged_workspace_bytes(2, 4, 1, 128, 8, 4)
    assert need == 4 * 2 * 4 * 1 * 4 * (128 + 1)
    assert call(splits=4) == c["ATTN_ERR_WORKSPACE"]
    assert call(splits=4, ws=FAKE, ws_bytes=need - 4) == c["ATTN_ERR_WORKSPACE"]


def test_paged_gqa_rejects_bad_arguments(api):
    c = header_constants()
    L = api.lib

    def call(Hq=8, Hkv=2, q_len=1, splits=1, ws=None, ws_bytes=0, o=FAKE):
        return L.attn_paged_decode_gqa(FAKE, FAKE, FAKE, FAKE, FAKE, o, None, 2, Hq, Hkv, q_len, 128,
                                       10, 8, 16, 1, 0.1, splits, ws, ws_bytes, 1, None)

    assert call(Hq=6, Hkv=4) == c["ATTN_ERR_BAD_SHAPE"]
    assert call(Hkv=0) == c["ATTN_ERR_BAD_SHAPE"]
    assert call(Hq=34, Hkv=2, q_len=1) == c["ATTN_ERR_UNSUPPORTED"]  # 17 query columns > 16
    assert call(Hq=16, Hkv=2, q_len=3) == c["ATTN_ERR_UNSUPPORTED"]  # 8 x 3 query columns > 16
    assert call(o=FAKE_ODD) == c["ATTN_ERR_MISALIGNED"]
    need = L.attn_paged_gqa_workspace_bytes(2, 8, 2, 1, 128, 8, 4)
    assert need == 4 * 2 * 8 * 1 * 4 * (128 + 1)
    assert call(splits=4) == c["ATTN_ERR_WORKSPACE"]
    assert call(splits=4, ws=FAKE, ws_bytes=need - 4) == c["ATTN_ERR_WORKSPACE"]
    assert L.attn_paged_gqa_workspace_bytes(2, 8, 3, 1, 128, 8, 4) == 0
    # equal head counts reproduce the ungrouped size
    assert L.attn_paged_gqa_workspace_bytes(2, 4, 4, 1, 128, 8, 4) == L.attn_paged_workspace_bytes(2, 4, 1, 128, 8, 4)


def test_paged_prefill_rejects_bad_arguments(api):
    c = header_constants()
    L = api.lib

    def call(q=FAKE, o=FAKE, B=2, H=4, q_len=64, D=128, nblk=10, width=8, bs=16, causal=1,
             scale=0.1, dtype=1):
        return L.attn_paged_prefill(q, FAKE, FAKE, FAKE, FAKE, o, None, B, H, q_len, D, nblk,
                                    width, bs, causal, scale, dtype, None)

    assert call(q=None) == c["ATTN_ERR_NULL_PTR"]
    assert call(q_len=0) == c["ATTN_ERR_BAD_SHAPE"]
    assert call(q_len=8 * 16 + 1) == c["ATTN_ERR_BAD_SHAPE"]  # longer than the table can hold
    assert call(dtype=0) == c["ATTN_ERR_BAD_DTYPE"]
    assert call(D=96) == c["ATTN_ERR_UNSUPPORTED"]
    assert call(bs=8) == c["ATTN_ERR_UNSUPPORTED"]
    assert call(width=2049) == c["ATTN_ERR_UNSUPPORTED"]  # ATTN_PAGED_PREFILL_MAX_BLOCKS + 1
    assert call(causal=2) == c["ATTN_ERR_BAD_SHAPE"]
    assert call(scale=float("inf")) == c["ATTN_ERR_BAD_SHAPE"]
    assert call(o=FAKE_ODD) == c["ATTN_ERR_MISALIGNED"]


def test_workspace_bytes(api):
    L = api.lib
    assert L.attn_paged_workspace_bytes(4, 40, 5, 128, 2048, 16) == 4 * 4 * 40 * 5 * 16 * 129
    assert L.attn_paged_workspace_bytes(4, 40, 5, 128, 2048, 1) == 0
    assert L.attn_paged_workspace_bytes(0, 40, 5, 128, 2048, 16) == 0
    assert L.attn_paged_workspace_bytes(4, 40, 17, 128, 2048, 16) == 0
    # automatic split count: about 128 blocks per split for batches of up to 64
    # sequences (run longest first), 32 for larger ones, raised towards 2048
    # (split, head, sequence) items while every split keeps >= 4 blocks
    assert L.attn_paged_workspace_bytes(1, 1, 1, 128, 15, 0) == 4 * 3 * 129
    assert L.attn_paged_workspace_bytes(1, 1, 1, 128, 3, 0) == 0
    assert L.attn_paged_workspace_bytes(1, 1, 1, 128, 256, 0) == 4 * 64 * 129
    # the 64-sequence x 40-head decode shape with 256-block tables: 2 splits;
    # one sequence more: 8 splits of 32 blocks
    assert L.attn_paged_workspace_bytes(64, 40, 1, 128, 256, 0) == 4 * 64 * 40 * 2 * 129
    assert L.attn_paged_workspace_bytes(65, 40, 1, 128, 256, 0) == 4 * 65 * 40 * 8 * 129
    # long sequences, few of them: 2048-block tables, 4 x 40 heads -> 16 splits
    assert L.attn_paged_workspace_bytes(4, 40, 5, 128, 2048, 0) == 4 * 4 * 40 * 5 * 16 * 129
    # grouped-query heads (8 query heads per KV head): about 256 blocks per
    # split, covering target 512 items: 64 x 8 KV heads of 256 blocks -> 1 split
    assert L.attn_paged_gqa_workspace_bytes(64, 64, 8, 1, 128, 256, 0) == 0
    assert L.attn_paged_gqa_workspace_bytes(4, 64, 8, 1, 128, 2048, 0) == 4 * 4 * 64 * 16 * 129


def test_merge_and_gather_reject_bad_arguments(api):
    c = header_constants()
    L = api.lib
    assert L.attn_lse_merge(None, FAKE, FAKE, None, 1, 1, 1, 2, 128, 1, None) == c["ATTN_ERR_NULL_PTR"]
    assert L.attn_lse_merge(FAKE, FAKE, FAKE, None, 1, 1, 1, 0, 128, 1, None) == c["ATTN_ERR_BAD_SHAPE"]
    assert L.attn_lse_merge(FAKE, FAKE, FAKE, None, 1, 1, 1, 2000, 128, 1, None) == c["ATTN_ERR_UNSUPPORTED"]
    assert L.attn_lse_merge(FAKE, FAKE, FAKE, None, 1, 1, 1, 2, 128, 5, None) == c["ATTN_ERR_BAD_DTYPE"]
    assert L.attn_paged_gather(FAKE, FAKE, FAKE, None, 1, 1, 128, 4, 4, 64, None) == c["ATTN_ERR_NULL_PTR"]
    assert L.attn_paged_gather(FAKE, FAKE, FAKE, FAKE, 1, 1, 100, 4, 4, 64, None) == c["ATTN_ERR_UNSUPPORTED"]
    assert L.attn_paged_gather(FAKE, FAKE, FAKE, FAKE, 1, 1, 128, 4, 4, 0, None) == c["ATTN_ERR_BAD_SHAPE"]


def test_check_tables_rejects_bad_arguments(api):
    c = header_constants()
    L = api.lib

    def call(tab=FAKE, lens=FAKE, B=2, min_len=1, nb=64, width=8, bad=FAKE):
        return L.attn_paged_check_tables(tab, lens, B, min_len, nb, width, bad, None)

    assert call(tab=None) == c["ATTN_ERR_NULL_PTR"]
    assert call(lens=None) == c["ATTN_ERR_NULL_PTR"]
    assert call(bad=None) == c["ATTN_ERR_NULL_PTR"]
    assert call(B=0) == c["ATTN_ERR_BAD_SHAPE"]
    assert call(min_len=-1) == c["ATTN_ERR_BAD_SHAPE"]
    assert call(nb=0) == c["ATTN_ERR_BAD_SHAPE"]
    assert call(width=0) == c["ATTN_ERR_BAD_SHAPE"]
    assert call(bad=ctypes.c_void_p((1 << 20) + 2)) == c["ATTN_ERR_MISALIGNED"]


def test_probe_is_a_library_of_its_own(api):
    """The benchmark's bandwidth probe is not part of the attention library."""
    assert not hasattr(api.lib, "attn_probe_block_read")
    assert "probe" not in " ".join(declared_functions())


def test_probe_rejects_bad_arguments():
    import probe
    L = probe.lib()

    def call(buf=FAKE, nb=64, bb=4096, order=FAKE, n=64, sink=FAKE, waves=8, nt=0):
        return L.probe_block_read(buf, nb, bb, order, n, sink, waves, nt, None)

    assert call(buf=None) == -1
    assert call(order=None) == -1
    assert call(sink=None) == -1
    assert call(nb=0) == -2
    assert call(n=0) == -2
    assert call(bb=3072) == -4
    assert call(bb=32768) == -4
    assert call(waves=6) == -2
    assert call(waves=0) == -2
    assert call(waves=1 << 23) == -2
    assert call(nt=2) == -2
    assert call(buf=FAKE_ODD) == -5
    assert call(order=ctypes.c_void_p((1 << 20) + 2)) == -5


def test_new_checks_reject_bad_arguments(api):
    c = header_constants()
    L = api.lib
    odd = ctypes.c_void_p((1 << 20) + 2)
    # append tables
    assert L.attn_paged_check_append(None, FAKE, 2, 3, 64, 8, FAKE, None) == c["ATTN_ERR_NULL_PTR"]
    assert L.attn_paged_check_append(FAKE, FAKE, 0, 3, 64, 8, FAKE, None) == c["ATTN_ERR_BAD_SHAPE"]
    assert L.attn_paged_check_append(FAKE, FAKE, 2, 0, 64, 8, FAKE, None) == c["ATTN_ERR_BAD_SHAPE"]
    assert L.attn_paged_check_append(FAKE, FAKE, 2, 3, 64, 8, odd, None) == c["ATTN_ERR_MISALIGNED"]
    # ragged offsets
    assert L.attn_paged_check_ragged(None, FAKE, 2, 40, 30, FAKE, None) == c["ATTN_ERR_NULL_PTR"]
    assert L.attn_paged_check_ragged(FAKE, FAKE, 2, 0, 30, FAKE, None) == c["ATTN_ERR_BAD_SHAPE"]
    assert L.attn_paged_check_ragged(FAKE, FAKE, 2, 40, 0, FAKE, None) == c["ATTN_ERR_BAD_SHAPE"]
    assert L.attn_paged_check_ragged(odd, FAKE, 2, 40, 30, FAKE, None) == c["ATTN_ERR_MISALIGNED"]
    # id lists
    assert L.attn_paged_check_ids(FAKE, None, 4, 64, FAKE, None) == c["ATTN_ERR_NULL_PTR"]
    assert L.attn_paged_check_ids(FAKE, FAKE, 0, 64, FAKE, None) == c["ATTN_ERR_BAD_SHAPE"]
    assert L.attn_paged_check_ids(FAKE, FAKE, 4, 0, FAKE, None) == c["ATTN_ERR_BAD_SHAPE"]
    assert L.attn_paged_check_ids(FAKE, odd, 4, 64, FAKE, None) == c["ATTN_ERR_MISALIGNED"]


def test_launch_size_limits(api):
    """Grids that the kernels could not be launched with are refused before
    anything is enqueued (a float32 prefill workgroup holds 4 query rows; the
    merge runs D threads per row, and a launch's work-items fit 32 bits)."""
    c = header_constants()
    L = api.lib
    # float32 prefill: 2^29 heads x 16 rows / 4 rows per workgroup = 2^31
    # workgroups, one past the limit (8 rows per workgroup would have passed)
    assert L.attn_prefill(FAKE, FAKE, FAKE, FAKE, None, 1 << 29, 1, 16, 64, 1, 0.1, 0, None) == \
        c["ATTN_ERR_OVERFLOW"]
    # merge: 2^25 rows x 128 threads = 2^32 work-items
    assert L.attn_lse_merge(FAKE, FAKE, FAKE, None, 1 << 25, 1, 1, 2, 128, 1, None) == \
        c["ATTN_ERR_OVERFLOW"]
    # paged decode with splits: the merge of 65535 x 65535 rows does not fit
    need = L.attn_paged_workspace_bytes(65535, 65535, 1, 128, 8, 2)
    assert L.attn_paged_decode(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 65535, 65535, 1, 128, 10,
                               8, 16, 1, 0.1, 2, FAKE, need, 1, None) == c["ATTN_ERR_OVERFLOW"]


def test_binding_refuses_cpu_tensors(api):
    import torch
    x = torch.zeros(1, 1, 4, 64)
    with pytest.raises(ValueError):
        api.attn_prefill(x, x, x)


def test_append_and_copy_reject_bad_arguments(api):
    c = header_constants()
    L = api.lib
    ok = dict(B=2, H=4, n=3, D=128, nb=16, W=4, bs=16, dtype=1)

    def app(k_new=FAKE, v_new=FAKE, kp=FAKE, vp=FAKE, bt=FAKE, sl=FAKE, **kw):
        a = dict(ok, **kw)
        return L.attn_paged_append(k_new, v_new, kp, vp, bt, sl, a["B"], a["H"], a["n"], a["D"],
                                   a["nb"], a["W"], a["bs"], a["dtype"], None)

    assert app(k_new=None) == c["ATTN_ERR_NULL_PTR"]
    assert app(sl=None) == c["ATTN_ERR_NULL_PTR"]
    assert app(n=0) == c["ATTN_ERR_BAD_SHAPE"]
    assert app(B=-1) == c["ATTN_ERR_BAD_SHAPE"]
    assert app(n=4 * 16 + 1) == c["ATTN_ERR_BAD_SHAPE"]  # more new tokens than a table can hold
    assert app(dtype=0) == c["ATTN_ERR_BAD_DTYPE"]
    assert app(D=96) == c["ATTN_ERR_UNSUPPORTED"]
    assert app(bs=32) == c["ATTN_ERR_UNSUPPORTED"]
    assert app(H=70000) == c["ATTN_ERR_OVERFLOW"]
    assert app(B=60000, H=60000, n=1 << 30, W=1 << 27) == c["ATTN_ERR_OVERFLOW"]
    assert app(kp=FAKE_ODD) == c["ATTN_ERR_MISALIGNED"]

    def cp(kp=FAKE, vp=FAKE, s=FAKE, d=FAKE, n=2, nb=16, H=4, D=128, dtype=1):
        return L.attn_paged_copy_blocks(kp, vp, s, d, n, nb, H, D, dtype, None)

    assert cp(s=None) == c["ATTN_ERR_NULL_PTR"]
    assert cp(n=0) == c["ATTN_ERR_BAD_SHAPE"]
    assert cp(dtype=0) == c["ATTN_ERR_BAD_DTYPE"]
    assert cp(D=32) == c["ATTN_ERR_UNSUPPORTED"]
    assert cp(n=70000) == c["ATTN_ERR_OVERFLOW"]
    assert cp(vp=FAKE_ODD) == c["ATTN_ERR_MISALIGNED"]


def test_paged_prefill_varlen_rejects_bad_arguments(api):
    c = header_constants()
    L = api.lib
    ok = dict(B=2, H=4, total=40, maxq=30, D=128, nb=64, W=8, bs=16, causal=1, dtype=1)

    def call(q=FAKE, cu=FAKE, o=FAKE, **kw):
        a = dict(ok, **kw)
        return L.attn_paged_prefill_varlen(q, FAKE, FAKE, FAKE, FAKE, cu, o, None, a["B"], a["H"],
                                           a["total"], a["maxq"], a["D"], a["nb"], a["W"],
                                           a["bs"], a["causal"], 0.1, a["dtype"], None)

    assert call(cu=None) == c["ATTN_ERR_NULL_PTR"]
    assert call(o=None) == c["ATTN_ERR_NULL_PTR"]
    assert call(total=0) == c["ATTN_ERR_BAD_SHAPE"]
    assert call(maxq=41) == c["ATTN_ERR_BAD_SHAPE"]          # longer than all queries together
    assert call(maxq=200, total=400) == c["ATTN_ERR_BAD_SHAPE"]  # past the table's 128 keys
    assert call(causal=2) == c["ATTN_ERR_BAD_SHAPE"]
    assert call(dtype=0) == c["ATTN_ERR_BAD_DTYPE"]
    assert call(D=80) == c["ATTN_ERR_UNSUPPORTED"]
    assert call(W=2049) == c["ATTN_ERR_UNSUPPORTED"]
    assert call(cu=ctypes.c_void_p((1 << 20) + 2)) == c["ATTN_ERR_MISALIGNED"]
    assert call(q=FAKE_ODD) == c["ATTN_ERR_MISALIGNED"]


def test_paged_prefill_gqa_rejects_bad_arguments(api):
    c = header_constants()
    L = api.lib

    def call(H=8, Hkv=2, q=FAKE, **kw):
        a = dict(dict(B=2, total=40, maxq=30, D=128, nb=64, W=8), **kw)
        return L.attn_paged_prefill_gqa(q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, a["B"], H,
                                        Hkv, a["total"], a["maxq"], a["D"], a["nb"], a["W"], 16,
                                        1, 0.1, 1, None)

    assert call(q=None) == c["ATTN_ERR_NULL_PTR"]
    assert call(Hkv=3) == c["ATTN_ERR_BAD_SHAPE"]       # 3 does not divide 8
    assert call(Hkv=0) == c["ATTN_ERR_BAD_SHAPE"]
    assert call(D=96) == c["ATTN_ERR_UNSUPPORTED"]
    assert call(q=FAKE_ODD) == c["ATTN_ERR_MISALIGNED"]


def test_binding_exports_what_it_lists(api):
    for name in api.__all__:
        assert hasattr(api, name), name


def test_noalloc_decode_refuses_partials_beyond_its_scratch(api):
    """attn_paged_decode_noalloc refuses, before anything touches a device,
    a call whose split-KV partials exceed the static scratch, and matches the
    binding's constant for its size."""
    c = header_constants()
    L = api.lib
    text = open(HEADER).read()
    m = re.search(r"#define ATTN_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == api.ATTN_NOALLOC_SCRATCH_BYTES
    limit = api.ATTN_NOALLOC_SCRATCH_BYTES

    def call(B, Hq, Hkv, q_len, W, S, q=FAKE, o=FAKE):
        return L.attn_paged_decode_noalloc(q, FAKE, FAKE, FAKE, FAKE, o, None, B, Hq, Hkv,
                                           q_len, 128, 64, W, 16, 1, 0.1, S, 1, None)

    assert call(64, 40, 40, 1, 256, 8, q=None) == c["ATTN_ERR_NULL_PTR"]
    # 64 sequences x 40 heads x 16 queries x 64 splits x 129 floats: 676 MB
    big = L.attn_paged_gqa_workspace_bytes(64, 40, 40, 16, 128, 4096, 64)
    assert big > limit
    assert call(64, 40, 40, 16, 4096, 64) == c["ATTN_ERR_SCRATCH"]
    # grouped-query: 8 query heads per KV head, q_len 2, 64 splits
    assert L.attn_paged_gqa_workspace_bytes(512, 64, 8, 2, 128, 4096, 64) > limit
    assert call(512, 64, 8, 2, 4096, 64) == c["ATTN_ERR_SCRATCH"]
    # the boundary: the largest split count whose partials still fit is not
    # refused for size; it fails later, at the device lookup (no GPU) or on
    # the misaligned output pointer, so that nothing is ever launched
    B, H, q_len = 64, 40, 4
    per_split = L.attn_paged_gqa_workspace_bytes(B, H, H, q_len, 128, 4096, 2) // 2
    s_fit = limit // per_split
    assert 2 <= s_fit < 64
    assert call(B, H, H, q_len, 4096, s_fit + 1) == c["ATTN_ERR_SCRATCH"]
    assert call(B, H, H, q_len, 4096, s_fit, o=FAKE_ODD) in (c["ATTN_ERR_HIP"],
                                                             c["ATTN_ERR_MISALIGNED"])


def test_library_imports_no_device_allocator(api):
    """The library never allocates device or host memory through HIP: none of
    HIP's allocation, free or memset routines is among its imports (the static
    scratch of attn_paged_decode_noalloc comes with the code object)."""
    import subprocess
    out = subprocess.run(["nm", "-D", "--undefined-only", api.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    hip = sorted({ln.split()[-1].split("@")[0] for ln in out.splitlines() if "hip" in ln})
    assert "hipGetSymbolAddress" in hip
    bad = [n for n in hip if re.search(r"Malloc|Free|Alloc|Memset|MemPool|HostRegister", n)]
    assert not bad, bad
