"""GPU parity of QK-Clip (mla_qk_clip) and the QK-Clip stress workload end to end."""

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib(gpu_available):
    import mla_qk_clip_amd as m
    return m


def _ulp_bf16(x):
    """Spacing of bf16 values at |x| (8 significant bits)."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, 2.0 ** (e - 7), 2.0 ** -133)


@pytest.mark.parametrize("bf16", [True, False])
def test_clip_threshold_and_rescale_match_oracle(lib, bf16):
    import torch
    import mla_qk_clip_amd as m
    from tests._gpu import dev, host, lib_dims, log
    dims = synth.Dims(8, 64, 16, 32, 24)
    D, NV = 48, 56
    rng = np.random.default_rng(41)
    wq = rng.standard_normal((8 * D, 40)).astype(np.float32)
    wk = rng.standard_normal((8 * NV, 64)).astype(np.float32)
    if bf16:
        wq, wk = synth.round_bf16(wq), synth.round_bf16(wk)
    tau = 50.0
    sm = np.array([tau - 1e-3, tau, np.nextafter(np.float32(tau), np.float32(1e9)), -np.inf, 1e4, 51.0, 0.0, -3.0],
                  dtype=np.float32)
    log(f"clip unit bf16={bf16}")
    wq_d, wk_d = dev(wq, bf16), dev(wk, bf16)
    clipped, gamma = m.mla_qk_clip(lib_dims(dims), wq_d, wk_d, torch.from_numpy(sm).cuda(), tau)
    torch.cuda.synchronize()
    rq, rk, mask, gm = oracle.qk_clip(wq, wk, sm.astype(np.float64), tau, dims)
    assert list(clipped.cpu().numpy().astype(bool)) == list(mask)
    assert list(mask) == [False, False, True, False, True, True, False, False]
    assert np.allclose(gamma.cpu().numpy(), gm, rtol=1e-6)
    gq, gk = host(wq_d), host(wk_d)
    if bf16:
        assert np.all(np.abs(gq - rq) <= _ulp_bf16(rq))
        assert np.all(np.abs(gk - rk) <= _ulp_bf16(rk))
    else:
        assert np.allclose(gq, rq, rtol=3e-7, atol=0) and np.allclose(gk, rk, rtol=3e-7, atol=0)
    for h in range(8):
        if not mask[h]:
            assert np.array_equal(gq[h * D:(h + 1) * D], wq[h * D:(h + 1) * D].astype(np.float64))
            assert np.array_equal(gk[h * NV:(h + 1) * NV], wk[h * NV:(h + 1) * NV].astype(np.float64))
        # V rows never written
        assert np.array_equal(gk[h * NV + 32:(h + 1) * NV], wk[h * NV + 32:(h + 1) * NV].astype(np.float64))


def _q_of(cq, wq, dims):
    """q = c^Q W_UQ (the query projection of the caller), bf16-rounded; input preparation."""
    q = cq.astype(np.float32) @ wq.astype(np.float32).T
    return synth.round_bf16(q).reshape(cq.shape[0], dims.heads, dims.nope_dim + dims.shared_dim)


def test_clip_stress_workload_end_to_end(lib):
    """Six heads with x40 query/key blocks exceed tau = 100 (logits > 1000); the
    clip mask is exactly those heads for both the GPU and the oracle; the
    rescaled weights match the oracle's to one bf16 ulp; after re-projecting
    the queries with the clipped weights every head's max logit is <= tau."""
    import torch
    import mla_qk_clip_amd as m
    from tests._gpu import dev, host, lib_dims, log, run_prefill
    p = synth.k3_clip_stress()
    dims = p.dims
    tau = synth.TAU
    log("clip stress: q projection")
    q = _q_of(p.cq, p.w_q_b, dims)
    log("clip stress: GPU prefill")
    _, _, ml = run_prefill(p, q=q, want_lse=False)
    sm = host(ml)
    log("clip stress: oracle max logits")
    ref_sm = np.array([oracle.max_logit_head(q, p.ckv, p.ks, p.w_kv_b, p.cu_seqlens, dims, h)
                       for h in range(dims.heads)])
    assert np.all(np.abs(sm - ref_sm) / np.abs(ref_sm) <= 1e-3)
    assert list(np.nonzero(sm > tau)[0]) == list(synth.CLIP_HEADS)
    assert list(np.nonzero(ref_sm > tau)[0]) == list(synth.CLIP_HEADS)
    assert sm[list(synth.CLIP_HEADS)].min() > 1000.0

    wq_d, wk_d = dev(p.w_q_b, True), dev(p.w_kv_b, True)
    clipped, gamma = m.mla_qk_clip(lib_dims(dims), wq_d, wk_d, ml, tau)
    torch.cuda.synchronize()
    assert list(np.nonzero(clipped.cpu().numpy())[0]) == list(synth.CLIP_HEADS)
    rq, rk, mask, gm = oracle.qk_clip(p.w_q_b, p.w_kv_b, ref_sm, tau, dims)
    gq, gk = host(wq_d), host(wk_d)
    assert np.all(np.abs(gq - rq) <= _ulp_bf16(rq))
    assert np.all(np.abs(gk - rk) <= _ulp_bf16(rk))
    D, NV = 192, 256
    for h in range(dims.heads):
        if h not in synth.CLIP_HEADS:
            assert np.array_equal(gq[h * D:(h + 1) * D], p.w_q_b[h * D:(h + 1) * D])
            assert np.array_equal(gk[h * NV:h * NV + 128], p.w_kv_b[h * NV:h * NV + 128])
        assert np.array_equal(gk[h * NV + 128:(h + 1) * NV], p.w_kv_b[h * NV + 128:(h + 1) * NV])

    log("clip stress: re-run with clipped weights")
    q2 = _q_of(p.cq, gq.astype(np.float32), dims)
    p2 = synth.PrefillInputs(dims, p.cu_seqlens, q2, p.ckv, p.ks, gk.astype(np.float32), p.gate, True)
    _, _, ml2 = run_prefill(p2, want_lse=False)
    sm2 = host(ml2)
    assert np.all(sm2 <= tau * (1 + 1e-3)), sm2.max()
    assert np.all(np.abs(sm2[list(synth.CLIP_HEADS)] - tau) <= 2e-2 * tau)
    others = [h for h in range(dims.heads) if h not in synth.CLIP_HEADS]
    assert np.array_equal(sm2[others], sm[others])
    del gamma, mask, gm
