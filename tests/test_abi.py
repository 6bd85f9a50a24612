"""The C-ABI library loads, exports every symbol include/mla.h declares, and
rejects bad arguments with status codes before launching anything (no GPU
needed: every case here fails validation on the host)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "mla.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def m():
    import mla_qk_clip_amd
    return mla_qk_clip_amd


def test_every_declared_symbol_is_exported(m):
    names = _declared()
    assert "mla_prefill" in names and "mla_absorbed" in names and "mla_qk_clip" in names
    for n in names:
        assert hasattr(m.lib, n), n
    assert set(names) == set(m.EXPORTED)


def test_version_and_status_strings(m):
    assert b"gfx950" in m.lib.mla_version()
    for s in range(5):
        assert m.lib.mla_status_string(s)


def _prefill(m, dims, **kw):
    args = dict(in_dt=m.MLA_BF16, out_dt=m.MLA_F32, q=16, ckv=16, ks=16, w=16, gate=None, qn=None, cu=16, nseq=1,
                ntok=10, out=16, lse=None, ml=16, acc=0, ws=16, wsb=1 << 40)
    args.update(kw)
    d = dims.c()
    return m.lib.mla_prefill(ctypes.byref(d), args["in_dt"], args["out_dt"], args["q"], args["ckv"], args["ks"],
                             args["w"], args["gate"], args["qn"], args["cu"], args["nseq"], args["ntok"], args["out"],
                             args["lse"], args["ml"], args["acc"], args["ws"], args["wsb"], None)


def test_prefill_validation(m):
    K3 = m.Dims()
    assert _prefill(m, K3, ml=None) == m.MLA_ERR_INVALID
    assert b"max_logit" in m.lib.mla_last_error()
    assert _prefill(m, K3, q=None) == m.MLA_ERR_INVALID
    assert _prefill(m, K3, q=24) == m.MLA_ERR_INVALID            # misaligned
    assert b"aligned" in m.lib.mla_last_error()
    assert _prefill(m, K3, ws=16, wsb=10) == m.MLA_ERR_WORKSPACE
    assert _prefill(m, K3, acc=2) == m.MLA_ERR_INVALID
    assert _prefill(m, K3, nseq=0) == m.MLA_ERR_INVALID
    assert _prefill(m, K3, ntok=-1) == m.MLA_ERR_INVALID
    assert _prefill(m, K3, in_dt=7) == m.MLA_ERR_INVALID
    assert _prefill(m, K3, in_dt=m.MLA_F32, out_dt=m.MLA_BF16) == m.MLA_ERR_UNSUPPORTED
    assert _prefill(m, m.Dims(96, 256, 64, 128, 128)) == m.MLA_ERR_UNSUPPORTED   # bf16 shape not compiled
    assert _prefill(m, m.Dims(0, 512, 64, 128, 128)) == m.MLA_ERR_INVALID
    assert _prefill(m, m.Dims(4, 2048, 16, 32, 32), in_dt=m.MLA_F32) == m.MLA_ERR_UNSUPPORTED
    assert m.lib.mla_prefill(None, 1, 0, None, None, None, None, None, None, None, 1, 1, None, None, None, 0, None,
                             0, None) == m.MLA_ERR_INVALID
    # the QK-norm argument: eps finite and >= 0, weight aligned
    qn = lambda w, eps: ctypes.pointer(m.mla_qk_norm(w, eps))  # noqa: E731
    assert _prefill(m, K3, qn=qn(None, -1.0)) == m.MLA_ERR_INVALID
    assert b"eps" in m.lib.mla_last_error()
    assert _prefill(m, K3, qn=qn(None, float("inf"))) == m.MLA_ERR_INVALID
    assert _prefill(m, K3, qn=qn(8, 1e-6)) == m.MLA_ERR_INVALID
    assert b"q_norm weight" in m.lib.mla_last_error()
    assert _prefill(m, K3, qn=qn(16, 1e-6), ws=16, wsb=10) == m.MLA_ERR_WORKSPACE   # a valid norm passes on


def test_absorbed_validation(m):
    K3 = m.Dims()
    d = K3.c()
    f = m.lib.mla_absorbed
    good = dict(q=16, cache=16, cap=100, lens=16, B=2, tq=1, w=16, gate=None, out=16, ml=16, acc=0, ws=16,
                wsb=1 << 40)

    def call(**kw):
        a = dict(good)
        a.update(kw)
        return f(ctypes.byref(d), m.MLA_BF16, m.MLA_BF16, a["q"], a["cache"], a["cap"], a["lens"], a["B"], a["tq"],
                 a["w"], a["gate"], a.get("qn"), a["out"], a["ml"], a["acc"], a["ws"], a["wsb"], None)
    assert call(tq=0) == m.MLA_ERR_INVALID
    assert call(cap=0) == m.MLA_ERR_INVALID
    assert call(lens=None) == m.MLA_ERR_INVALID
    assert call(wsb=5) == m.MLA_ERR_WORKSPACE
    assert call(gate=8) == m.MLA_ERR_INVALID
    big = m.Dims(200).c()
    assert f(ctypes.byref(big), m.MLA_BF16, m.MLA_BF16, 16, 16, 100, 16, 1, 1, 16, None, None, 16, 16, 0, 16,
             1 << 40, None) == m.MLA_ERR_UNSUPPORTED
    assert call(qn=ctypes.pointer(m.mla_qk_norm(None, -0.5))) == m.MLA_ERR_INVALID


def test_absorbed_noalloc_validation(m):
    """The no-allocation variant runs the same checks, then refuses sizes whose
    scratch would not fit its built-in 128 MiB, all before any HIP call."""
    d = m.Dims().c()
    f = m.lib.mla_absorbed_noalloc
    good = dict(q=16, cache=16, cap=100, lens=16, B=2, tq=1, w=16, gate=None, out=16, ml=16, acc=0)

    def call(**kw):
        a = dict(good)
        a.update(kw)
        return f(ctypes.byref(d), m.MLA_BF16, m.MLA_BF16, a["q"], a["cache"], a["cap"], a["lens"], a["B"], a["tq"],
                 a["w"], a["gate"], None, a["out"], a["ml"], a["acc"], None)
    assert call(tq=0) == m.MLA_ERR_INVALID
    assert call(lens=None) == m.MLA_ERR_INVALID
    assert call(ml=2) == m.MLA_ERR_INVALID
    assert call(acc=2) == m.MLA_ERR_INVALID
    limit = 128 << 20
    K3 = m.Dims()
    fits = max(b for b in range(1, 400) if m.mla_absorbed_workspace_size(K3, m.MLA_BF16, b, 1) <= limit)
    assert 160 <= fits <= 180
    assert call(B=fits + 1) == m.MLA_ERR_UNSUPPORTED
    assert b"built-in scratch" in m.lib.mla_last_error()
    assert call(B=fits // 2, tq=3) == m.MLA_ERR_UNSUPPORTED


def test_expanded_validation(m):
    K3 = m.Dims()
    d = K3.c()
    f = m.lib.mla_expanded
    good = dict(in_dt=m.MLA_BF16, q=16, k=16, v=16, cap=100, lens=16, B=2, tq=1, gate=None, out=16, ml=16, acc=0,
                ws=16, wsb=1 << 40)

    def call(**kw):
        a = dict(good)
        a.update(kw)
        return f(ctypes.byref(d), a["in_dt"], m.MLA_BF16, a["q"], a["k"], a["v"], a["cap"], a["lens"], a["B"],
                 a["tq"], a["gate"], a["out"], a["ml"], a["acc"], a["ws"], a["wsb"], None)
    assert call(in_dt=m.MLA_F32) == m.MLA_ERR_UNSUPPORTED
    assert call(tq=0) == m.MLA_ERR_INVALID
    assert call(cap=0) == m.MLA_ERR_INVALID
    assert call(cap=(1 << 27) + 1) == m.MLA_ERR_UNSUPPORTED
    assert call(k=None) == m.MLA_ERR_INVALID
    assert call(v=24) == m.MLA_ERR_INVALID
    assert b"aligned" in m.lib.mla_last_error()
    assert call(ml=None) == m.MLA_ERR_INVALID
    assert call(wsb=5) == m.MLA_ERR_WORKSPACE
    assert call(acc=3) == m.MLA_ERR_INVALID
    small = m.Dims(4, 256, 64, 128, 128).c()
    assert f(ctypes.byref(small), m.MLA_BF16, m.MLA_BF16, 16, 16, 16, 100, 16, 1, 1, None, 16, 16, 0, 16, 1 << 40,
             None) == m.MLA_ERR_UNSUPPORTED
    # per (query, head, split of 2048 rows): 128 outputs and {max, sum} in fp32
    assert m.mla_expanded_workspace_size(K3, m.MLA_BF16, 64, 1, 32768) >= 64 * 96 * 16 * 130 * 4
    assert m.mla_expanded_workspace_size(K3, m.MLA_F32, 64, 1, 32768) == 0


def test_linear_norm_layer_and_backward_validation(m):
    """The whole-layer blocks and the backward refuse bad sizes, dtypes and
    pointers on the host, before any launch."""
    K3 = m.Dims()
    d = K3.c()
    lin = m.lib.mla_linear
    assert lin(m.MLA_F32, 16, 4, 128, 16, 8, 16, None) == m.MLA_ERR_UNSUPPORTED
    assert lin(m.MLA_BF16, 16, 4, 96, 16, 8, 16, None) == m.MLA_ERR_UNSUPPORTED      # k not a multiple of 128
    assert lin(m.MLA_BF16, 16, 4, 128, 16, 12, 16, None) == m.MLA_ERR_UNSUPPORTED    # n not a multiple of 8
    assert lin(m.MLA_BF16, None, 4, 128, 16, 8, 16, None) == m.MLA_ERR_INVALID
    assert lin(m.MLA_BF16, 24, 4, 128, 16, 8, 16, None) == m.MLA_ERR_INVALID         # misaligned
    assert lin(m.MLA_BF16, None, 0, 128, None, 8, None, None) == m.MLA_OK            # nothing to do
    nrm = m.lib.mla_rms_norm
    assert nrm(m.MLA_BF16, 16, 4, 4096, 16, 1e-6, 16, None) == m.MLA_ERR_UNSUPPORTED  # wider than 2048
    assert nrm(m.MLA_BF16, 16, 4, 512, 16, -1.0, 16, None) == m.MLA_ERR_INVALID
    assert nrm(m.MLA_BF16, 16, 4, 512, None, 1e-6, 16, None) == m.MLA_ERR_INVALID
    lay = m.lib.mla_layer_forward

    def layer(hidden=256, q_rank=128, eps=1e-6, x=16, out=16, ml=16, ws=16, wsb=1 << 40):
        return lay(ctypes.byref(d), hidden, q_rank, eps, x, 16, 16, 16, 16, 16, 16, 16, 16, 16, 1, 10, out, ml, 0,
                   ws, wsb, None)
    assert layer(hidden=200) == m.MLA_ERR_UNSUPPORTED
    assert layer(q_rank=4096) == m.MLA_ERR_UNSUPPORTED
    assert layer(eps=float("nan")) == m.MLA_ERR_INVALID
    assert layer(x=None) == m.MLA_ERR_INVALID
    assert layer(ml=None) == m.MLA_ERR_INVALID
    assert layer(wsb=16) == m.MLA_ERR_WORKSPACE
    assert m.mla_layer_workspace_size(K3, 7168, 1536, 4096, 1) > 4096 * (1536 + 576 + 12288 + 18432) * 2
    bwd = m.lib.mla_prefill_backward

    def back(cu_=16, nseq=2, T=10, dq=16, gate=None, dgate=None, wsb=1 << 40):
        return bwd(ctypes.byref(d), 16, 16, 16, 16, gate, cu_, nseq, T, 16, 16, 16, dq, 16, 16, 16, dgate, 16, wsb,
                   None)
    assert back(cu_=None) == m.MLA_ERR_INVALID
    assert back(cu_=18) == m.MLA_ERR_INVALID        # cu_seqlens (int32) misaligned
    assert back(nseq=0) == m.MLA_ERR_INVALID        # tokens need a sequence
    assert back(nseq=-1) == m.MLA_ERR_INVALID
    assert back(dq=None) == m.MLA_ERR_INVALID
    assert back(gate=16, dgate=None) == m.MLA_ERR_INVALID   # a gate needs its gradient buffer
    assert back(wsb=16) == m.MLA_ERR_WORKSPACE
    assert back(T=0) == m.MLA_OK
    assert back(T=(1 << 20) + 1) == m.MLA_ERR_UNSUPPORTED
    # O(T H) workspace: linear in the token count, independent of the sequence lengths
    ws = m.lib.mla_prefill_backward_workspace_size
    for t in (4096, 8192, 65536):
        # about 2 KB per token and head, plus split-K partials of at most 256 MB
        assert t * 96 * 1024 < ws(ctypes.byref(d), t, 1) < t * 96 * 2200 + (1 << 28)
    w4 = ws(ctypes.byref(d), 4096, 1)
    assert ws(ctypes.byref(d), 4096, 64) - w4 < 4096
    assert ws(ctypes.byref(d), 4096, -1) == 0


def test_qk_clip_validation(m):
    K3 = m.Dims()
    d = K3.c()
    f = m.lib.mla_qk_clip
    assert f(ctypes.byref(d), m.MLA_BF16, 16, 1536, 16, 16, 0.0, None, None, None) == m.MLA_ERR_INVALID
    assert f(ctypes.byref(d), m.MLA_BF16, 16, 1536, 16, 16, float("nan"), None, None, None) == m.MLA_ERR_INVALID
    assert f(ctypes.byref(d), m.MLA_BF16, 16, 1530, 16, 16, 100.0, None, None, None) == m.MLA_ERR_UNSUPPORTED
    assert f(ctypes.byref(d), m.MLA_BF16, None, 1536, 16, 16, 100.0, None, None, None) == m.MLA_ERR_INVALID
    assert f(ctypes.byref(d), m.MLA_BF16, 16, 1536, 16, None, 100.0, None, None, None) == m.MLA_ERR_INVALID


def test_workspace_sizes(m):
    K3 = m.Dims()
    a = m.mla_prefill_workspace_size(K3, m.MLA_BF16, 4096, 1)
    b = m.mla_prefill_workspace_size(K3, m.MLA_BF16, 59392, 4)
    # expanded K^C and V^T of every head dominate: 96 heads x 256 values x 2 bytes per padded row
    assert a >= 96 * 256 * 2 * 4096 and b >= 96 * 256 * 2 * 59392
    assert m.mla_absorbed_workspace_size(K3, m.MLA_BF16, 64, 1) > 0
    assert m.mla_prefill_workspace_size(m.Dims(0), m.MLA_BF16, 10, 1) == 0


def test_binding_rejects_host_tensors_before_any_launch(m):
    """The binding checks every tensor against the sizes it passes to the C ABI
    (which takes bare pointers): host tensors are refused before any call."""
    import torch
    d = m.Dims(heads=2, kv_rank=16, shared_dim=8, nope_dim=8, v_dim=8)
    T = 5
    q = torch.zeros((T, 2, 16), dtype=torch.float32)
    ckv, ks = torch.zeros((T, 16)), torch.zeros((T, 8))
    w = torch.zeros((2 * 16, 16))
    cu = torch.tensor([0, T], dtype=torch.int32)
    with pytest.raises(ValueError, match="device tensor"):
        m.mla_prefill(d, q, ckv, ks, w, None, cu)
    with pytest.raises(ValueError, match="device tensor"):
        m.mla_absorbed(d, q[None, :1], torch.zeros((1, 8, 24)), torch.tensor([8], dtype=torch.int32), w, None)
    K3 = m.Dims(heads=2)
    with pytest.raises(ValueError, match="device tensor"):
        m.mla_expanded(K3, torch.zeros((1, 1, 2, 192), dtype=torch.bfloat16),
                       torch.zeros((1, 2, 8, 192), dtype=torch.bfloat16), torch.zeros((1, 2, 8, 128), dtype=torch.bfloat16),
                       torch.tensor([8], dtype=torch.int32), None)
