"""CPU checks of the Python binding's argument validation.

The binding must refuse, before any launch, output and workspace tensors that
do not match what the kernels will write: a short `o`, `lse` or `out` would be
written past its end. Here the device type the binding accepts is switched to
"cpu" and the library is replaced by a stub that records calls, so the checks
run without a GPU and a call that passes them is seen, not launched.
"""

import pytest
import torch


class StubLib:
    def __init__(self, real):
        self.calls = []
        self._real = real

    def __getattr__(self, name):
        if name.startswith("attn_") and name not in ("attn_status_string", "attn_version") \
                and not name.endswith("_workspace_bytes"):
            def rec(*args):
                self.calls.append(name)
                return 0
            return rec
        return getattr(self._real, name)


@pytest.fixture
def api(monkeypatch):
    import attention_tiled_qk_amd as m
    stub = StubLib(m.lib)
    monkeypatch.setattr(m, "_DEVICE_TYPE", "cpu")
    monkeypatch.setattr(m, "lib", stub)
    monkeypatch.setattr(m, "_stream", lambda device, stream: None)
    return m, stub


def bf(*shape):
    return torch.zeros(*shape, dtype=torch.bfloat16)


def i32(*shape):
    return torch.zeros(*shape, dtype=torch.int32)


def test_prefill_outputs_must_match(api):
    m, stub = api
    q = bf(2, 3, 40, 64)
    m.attn_prefill(q, q.clone(), q.clone(), causal=True)
    assert stub.calls == ["attn_prefill"]
    with pytest.raises(ValueError, match="o must have shape"):
        m.attn_prefill(q, q, q, o=bf(2, 3, 39, 64))
    with pytest.raises(ValueError, match="lse must have shape"):
        m.attn_prefill(q, q, q, lse=torch.zeros(2, 3, 20))
    with pytest.raises(ValueError, match="k must have shape"):
        m.attn_prefill(q, bf(2, 3, 41, 64), q)
    with pytest.raises(ValueError, match="must be torch.float32"):
        m.attn_prefill(q, q, q, lse=torch.zeros(2, 3, 40, dtype=torch.float64))
    assert stub.calls == ["attn_prefill"]


def paged(B=3, H=4, q_len=2, D=128, nblk=20, W=6):
    return (bf(B, H, q_len, D), bf(nblk, H, 16, D), bf(nblk, H, 16, D), i32(B, W), i32(B))


def test_paged_decode_outputs_and_workspace(api):
    m, stub = api
    q, kp, vp, bt, sl = paged()
    m.attn_paged_decode(q, kp, vp, bt, sl, num_splits=1)
    assert stub.calls == ["attn_paged_decode"]
    with pytest.raises(ValueError, match="o must have shape"):
        m.attn_paged_decode(q, kp, vp, bt, sl, o=bf(3, 4, 1, 128))
    with pytest.raises(ValueError, match="lse must have shape"):
        m.attn_paged_decode(q, kp, vp, bt, sl, lse=torch.zeros(3, 4))
    need = m.attn_paged_workspace_bytes(3, 4, 2, 128, 6, 2)
    assert need > 0
    with pytest.raises(ValueError, match="workspace holds"):
        m.attn_paged_decode(q, kp, vp, bt, sl, num_splits=2,
                            workspace=torch.zeros(need // 4 - 1, dtype=torch.float32))
    with pytest.raises(TypeError):
        m.attn_paged_decode(q, kp, vp, bt, sl, num_splits=2, workspace=12345)
    with pytest.raises(ValueError, match="contiguous"):
        ws = torch.zeros(2 * need, dtype=torch.uint8)[::2]
        m.attn_paged_decode(q, kp, vp, bt, sl, num_splits=2, workspace=ws)
    # a large enough workspace of any dtype is accepted
    m.attn_paged_decode(q, kp, vp, bt, sl, num_splits=2, workspace=torch.zeros(need, dtype=torch.uint8))
    assert stub.calls == ["attn_paged_decode", "attn_paged_decode"]


def test_paged_prefill_and_varlen_outputs(api):
    m, stub = api
    q, kp, vp, bt, sl = paged(q_len=5)
    with pytest.raises(ValueError, match="o must have shape"):
        m.attn_paged_prefill(q, kp, vp, bt, sl, o=bf(3, 4, 4, 128))
    with pytest.raises(ValueError, match="lse must have shape"):
        m.attn_paged_prefill(q, kp, vp, bt, sl, lse=torch.zeros(3, 4, 4))
    qv = bf(9, 4, 128)
    cu = torch.tensor([0, 4, 4, 9], dtype=torch.int32)
    with pytest.raises(ValueError, match="o must have shape"):
        m.attn_paged_prefill_varlen(qv, kp, vp, bt, sl, cu, 5, o=bf(8, 4, 128))
    with pytest.raises(ValueError, match="lse must have shape"):
        m.attn_paged_prefill_varlen(qv, kp, vp, bt, sl, cu, 5, lse=torch.zeros(9, 3))
    m.attn_paged_prefill_varlen(qv, kp, vp, bt, sl, cu, 5)
    assert stub.calls == ["attn_paged_prefill_varlen"]


def test_merge_gather_and_fp8_outputs(api):
    m, stub = api
    op = torch.zeros(2, 3, 1, 4, 64)
    lp = torch.zeros(2, 3, 1, 4)
    with pytest.raises(ValueError, match="o must have shape"):
        m.attn_lse_merge(op, lp, o=bf(2, 3, 1, 32))
    with pytest.raises(ValueError, match="lse must have shape"):
        m.attn_lse_merge(op, lp, lse=torch.zeros(2, 3))
    pool = bf(10, 2, 16, 64)
    with pytest.raises(ValueError, match="out must have shape"):
        m.attn_paged_gather(pool, i32(3, 4), i32(3), 64, out=bf(3, 2, 63, 64))
    q = bf(3, 8, 1, 128)
    kc = torch.zeros(10, 2, 16, 128, dtype=torch.uint8)
    sc = torch.zeros(10, 2)
    with pytest.raises(ValueError, match="o must have shape"):
        m.attn_paged_decode_fp8(q, kc, kc.clone(), sc, sc.clone(), i32(3, 4), i32(3),
                                o=bf(3, 8, 2, 128))
    with pytest.raises(ValueError, match="workspace holds"):
        m.attn_paged_decode_fp8(q, kc, kc.clone(), sc, sc.clone(), i32(3, 4), i32(3),
                                num_splits=2, workspace=torch.zeros(4))
    assert stub.calls == []
