"""GPU parity of the whole-layer path (mla_linear, mla_rms_norm,
mla_layer_forward) against the CPU oracle."""
import numpy as np
import pytest

import oracle
import synth
from tests._util import rel_err

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
SMAX_TOL = 1e-3
EPS = 1e-6


@pytest.fixture(scope="module")
def lib(gpu_available):
    import mla_qk_clip_amd as m
    return m


@pytest.mark.parametrize("m_,k,n", [(300, 384, 584), (1, 128, 8), (257, 7168, 256), (512, 1536, 2112)])
def test_linear_ragged_shapes(lib, m_, k, n):
    """Row and column counts that are not multiples of the 256 x 256 tile (one
    row; one column block of 8; a ragged tail of 72 columns), long K."""
    import mla_qk_clip_amd as m
    from tests._gpu import dev, host, log
    rng = np.random.default_rng(51)
    x = synth.round_bf16(rng.standard_normal((m_, k)).astype(np.float32))
    w = synth.round_bf16((rng.standard_normal((n, k)) / np.sqrt(k)).astype(np.float32))
    log(f"linear m={m_} k={k} n={n}")
    y = m.mla_linear(dev(x, True), dev(w, True))
    ref = oracle.linear(x, w)
    got = host(y)
    assert rel_err(got, ref) <= 8e-3          # one bf16 rounding of an fp32 sum
    assert np.all(np.isfinite(got))


@pytest.mark.parametrize("n", [1536, 512, 8])
def test_rms_norm(lib, n):
    import mla_qk_clip_amd as m
    from tests._gpu import dev, host, log
    rng = np.random.default_rng(52)
    x = synth.round_bf16((3.0 * rng.standard_normal((37, n))).astype(np.float32))
    w = synth.round_bf16((1.0 + 0.1 * rng.standard_normal(n)).astype(np.float32))
    log(f"rms_norm n={n}")
    y = m.mla_rms_norm(dev(x, True), dev(w, True), EPS)
    assert rel_err(host(y), oracle.rms_norm(x, w, EPS)) <= 8e-3


def _run_layer(L, **kw):
    import torch
    import mla_qk_clip_amd as m
    from tests._gpu import dev, dev_i32, lib_dims
    out, ml = m.mla_layer_forward(lib_dims(L.dims), dev(L.x, True), dev(L.w_dq, True), dev(L.g_q, True),
                                  dev(L.w_uq, True), dev(L.w_kv_a, True), dev(L.g_kv, True), dev(L.w_kv_b, True),
                                  dev(L.w_g, True), dev(L.w_o, True), dev_i32(L.cu_seqlens), eps=EPS, **kw)
    torch.cuda.synchronize()
    return out, ml


def test_layer_small_varlen(lib):
    """Four heads, hidden 256, q_rank 256, two sequences (70 and 129 tokens):
    the full output and every head's max logit."""
    from tests._gpu import host, log
    dims = synth.Dims(4, 512, 64, 128, 128)
    L = synth.layer_inputs(dims, 256, 256, [70, 129], seed=53, bf16=True)
    log("layer small varlen")
    out, ml = _run_layer(L)
    ref, ref_sm = oracle.layer_forward(L.x, L.w_dq, L.g_q, L.w_uq, L.w_kv_a, L.g_kv, L.w_kv_b, L.w_g, L.w_o,
                                       L.cu_seqlens, dims, EPS)
    assert rel_err(host(out), ref) <= BF16_TOL
    assert np.all(np.abs(host(ml) - ref_sm) / np.abs(ref_sm) <= SMAX_TOL)


def test_layer_accumulates_max_logit(lib):
    import torch
    from tests._gpu import host, log
    dims = synth.Dims(4, 512, 64, 128, 128)
    L = synth.layer_inputs(dims, 128, 128, [33], seed=54, bf16=True)
    log("layer accumulate")
    _, ml0 = _run_layer(L)
    prior = torch.tensor([1e3, -1e3, 1e3, -1e3], dtype=torch.float32, device="cuda")
    _, ml = _run_layer(L, max_logit=prior, accumulate=True)
    got, base = host(ml), host(ml0)
    assert got[0] == 1e3 and got[2] == 1e3 and got[1] == base[1] and got[3] == base[3]


def test_layer_k3_4096_sampled(lib):
    """The whole Kimi K3 layer (hidden 7168, q_lora_rank 1536, 96 heads) at
    T = 4096: sampled output rows against the oracle, and the max logit of
    three heads."""
    from tests._gpu import host, log
    L = synth.k3_layer()
    log("K3 layer T=4096: GPU")
    out, ml = _run_layer(L)
    rows = [0, 1, 63, 64, 1000, 2047, 4094, 4095]
    log("oracle rows")
    ref, q, ckv, ks = oracle.layer_rows(L.x, L.w_dq, L.g_q, L.w_uq, L.w_kv_a, L.g_kv, L.w_kv_b, L.w_g, L.w_o,
                                        L.cu_seqlens, L.dims, EPS, rows)
    got = host(out)
    assert np.all(np.isfinite(got))
    assert rel_err(got[rows], ref) <= BF16_TOL
    log("oracle max logits")
    sm = host(ml)
    for h in (0, 41, 95):
        want = oracle.max_logit_head(q, ckv, ks, L.w_kv_b, L.cu_seqlens, L.dims, h)
        assert abs(sm[h] - want) <= SMAX_TOL * abs(want), (h, sm[h], want)


def test_empty_inputs_only_reset_the_max_logit(lib):
    """Zero tokens (layer), zero sequences (expanded decode) and zero rows
    (linear) launch nothing but the max-logit reset."""
    import torch
    import mla_qk_clip_amd as m
    from tests._gpu import host, log
    log("empty inputs")
    dims = m.Dims(4)
    bf = dict(dtype=torch.bfloat16, device="cuda")
    ml = torch.full((4,), 7.0, dtype=torch.float32, device="cuda")
    w = lambda *s: torch.zeros(s, **bf)
    m.mla_layer_forward(dims, w(0, 256), w(128, 256), w(128), w(4 * 192, 128), w(576, 256), w(512), w(4 * 256, 512),
                        w(4 * 128, 256), w(256, 4 * 128), torch.zeros(1, dtype=torch.int32, device="cuda"),
                        max_logit=ml)
    torch.cuda.synchronize()
    assert np.all(host(ml) == -np.inf)
    ml.fill_(7.0)
    m.mla_expanded(dims, w(0, 1, 4, 192), w(0, 4, 8, 192), w(0, 4, 8, 128),
                   torch.zeros(0, dtype=torch.int32, device="cuda"), None, max_logit=ml)
    torch.cuda.synchronize()
    assert np.all(host(ml) == -np.inf)
    y = m.mla_linear(w(0, 128), w(8, 128))
    assert tuple(y.shape) == (0, 8)
