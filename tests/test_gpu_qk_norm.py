"""GPU parity of the QK-norm variant (a per-head RMSNorm of the queries, the
`q_norm` argument of mla_prefill and mla_absorbed) against the oracle, and the
clip-stress workload run with it: how far the norm alone brings the logits of
heads whose query and key weights are scaled x40.

Tolerances as for the plain calls: bf16 outputs <= 2e-2 normwise, fp32 <= 1e-4,
max logits <= 1e-3 relative.
"""
import numpy as np
import pytest

import oracle
import synth
from tests._util import rel_err

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
F32_TOL = 1e-4
SMAX_TOL = 1e-3
EPS = 1e-6


@pytest.fixture(scope="module")
def lib(gpu_available):
    import mla_qk_clip_amd as m
    return m


def _weight(D, seed, bf16):
    w = 1.0 + 0.1 * np.random.default_rng(seed).standard_normal(D).astype(np.float32)
    return synth.round_bf16(w) if bf16 else w


def _prefill(p, weight, out_dtype=None):
    import torch
    import mla_qk_clip_amd as m
    from tests._gpu import dev, dev_i32, lib_dims
    bf = p.bf16
    w = None if weight is None else dev(weight, bf)
    out, lse, ml = m.mla_prefill(lib_dims(p.dims), dev(p.q, bf), dev(p.ckv, bf), dev(p.ks, bf), dev(p.w_kv_b, bf),
                                 None if p.gate is None else dev(p.gate, bf), dev_i32(p.cu_seqlens),
                                 out_dtype=out_dtype or torch.float32, want_lse=True, q_norm=(w, EPS))
    torch.cuda.synchronize()
    return out, lse, ml


@pytest.mark.parametrize("with_weight", [True, False])
def test_qk_norm_bf16_prefill_varlen_matches_oracle(lib, with_weight):
    """Ragged sequences (empty, one token, across tile edges), queries of
    very different scales per head, a per-feature weight or none."""
    from tests._gpu import host, log
    dims = synth.Dims(8, 512, 64, 128, 128)
    p = synth.prefill_inputs(dims, [1, 63, 64, 65, 0, 130, 300, 7], seed=61, bf16=True)
    p.q = synth.round_bf16(p.q * np.array([1, 40, 0.02, 3, 1, 1, 7, 0.5], dtype=np.float32)[None, :, None])
    w = _weight(192, 62, True) if with_weight else None
    log(f"QK-norm bf16 prefill (weight={with_weight})")
    out, lse, ml = _prefill(p, w)
    ref, ref_lse, ref_sm = oracle.qk_norm_prefill(p.q, p.ckv, p.ks, p.w_kv_b, p.gate, p.cu_seqlens, dims, w, EPS)
    assert rel_err(host(out), ref) <= BF16_TOL
    n = p.ntok
    assert np.max(np.abs(host(lse)[:, :n] - ref_lse)) <= 1e-2
    sm = host(ml)
    assert np.all(np.abs(sm - ref_sm) / np.abs(ref_sm) <= SMAX_TOL), np.abs(sm - ref_sm) / np.abs(ref_sm)


def test_qk_norm_fp32_tiny_matches_oracle(lib):
    from tests._gpu import host, log
    p = synth.tiny_fp32_prefill()
    w = _weight(48, 63, False)
    log("QK-norm fp32 tiny prefill")
    out, lse, ml = _prefill(p, w)
    ref, ref_lse, ref_sm = oracle.qk_norm_prefill(p.q, p.ckv, p.ks, p.w_kv_b, p.gate, p.cu_seqlens, p.dims, w, EPS,
                                                  round_bf16=False)
    assert rel_err(host(out), ref) <= F32_TOL
    assert np.max(np.abs(host(lse) - ref_lse)) <= 1e-4
    assert np.all(np.abs(host(ml) - ref_sm) / np.abs(ref_sm) <= SMAX_TOL)


@pytest.mark.parametrize("tq", [1, 3])
def test_qk_norm_bf16_absorbed_matches_oracle(lib, tq):
    import torch
    import mla_qk_clip_amd as m
    from tests._gpu import decode_cache_tensor, dev, dev_i32, host, lib_dims, log
    d = synth.decode_inputs(synth.K3, [3000, 700, 5, 1500], cap=3008, tq=tq, seed=64, bf16=True)
    d.q = synth.round_bf16(d.q * np.linspace(0.05, 30, 96, dtype=np.float32)[None, None, :, None])
    w = _weight(192, 65, True)
    log(f"QK-norm bf16 absorbed tq={tq}")
    out, ml = m.mla_absorbed(lib_dims(d.dims), dev(d.q, True), decode_cache_tensor(d), dev_i32(d.lens),
                             dev(d.w_kv_b, True), dev(d.gate, True), out_dtype=torch.float32,
                             q_norm=(dev(w, True), EPS))
    torch.cuda.synchronize()
    rows = [d.cache_rows(b) for b in range(d.batch)]
    ref, ref_sm = oracle.qk_norm_absorbed(d.q, rows, d.w_kv_b, d.gate, d.dims, w, EPS)
    assert rel_err(host(out), ref) <= BF16_TOL
    assert np.all(np.abs(host(ml) - ref_sm) / np.abs(ref_sm) <= SMAX_TOL)


def test_qk_norm_fp32_absorbed_equals_fp32_prefill_last_rows(lib):
    import torch
    import mla_qk_clip_amd as m
    from tests._gpu import dev, dev_i32, host, lib_dims, log
    p = synth.tiny_fp32_prefill()
    w = _weight(48, 66, False)
    log("QK-norm fp32 absorbed vs prefill")
    out_p, _, _ = _prefill(p, w)
    cache = np.concatenate([p.ckv, p.ks], axis=1)[None]
    out_d, ml = m.mla_absorbed(lib_dims(p.dims), dev(p.q[None, -4:], False), dev(cache, False), dev_i32([64]),
                               dev(p.w_kv_b, False), dev(p.gate[None, -4:], False), q_norm=(dev(w, False), EPS))
    torch.cuda.synchronize()
    assert rel_err(host(out_d)[0], host(out_p)[-4:]) <= F32_TOL


def test_qk_norm_on_the_clip_stress_workload(lib):
    """The clip-stress recipe (T = 2048; heads 0, 19, 38, 57, 76, 95 with their
    q_b_proj rows and W_UK rows x40) with the QK-norm variant on. The norm
    takes out the query-side factor: those heads' max logits fall from above
    1000 to about 40 times an ordinary head's. It does not remove the key-side
    factor, which enters through W_UK between the normalised query and the
    normalised latent, so they stay above tau = 100 and the clip still fires;
    the other heads do not move."""
    from tests._gpu import host, log, run_prefill
    p = synth.k3_clip_stress()
    dims = p.dims
    log("clip stress with QK-norm: q projection")
    q = synth.round_bf16(p.cq.astype(np.float32) @ p.w_q_b.astype(np.float32).T).reshape(p.ntok, 96, 192)
    p.q = q
    log("GPU prefill without and with the norm")
    _, _, ml_plain = run_prefill(p, want_lse=False)
    _, _, ml_norm = _prefill(p, None)
    sm0, sm1 = host(ml_plain), host(ml_norm)
    heads = list(synth.CLIP_HEADS)
    others = [0 + h for h in (1, 20, 47, 94)]
    log("oracle max logits with the norm")
    qn = oracle.qk_norm_query(q, None, EPS)
    ref = {h: oracle.max_logit_head(qn, p.ckv, p.ks, p.w_kv_b, p.cu_seqlens, dims, h) for h in heads + others}
    for h, r in ref.items():
        assert abs(sm1[h] - r) / abs(r) <= SMAX_TOL, (h, sm1[h], r)
    assert sm0[heads].min() > 1000.0
    assert np.all(sm1[heads] > synth.TAU) and np.all(sm1[heads] < sm0[heads] / 20)
    assert np.all(np.abs(sm1[others] - sm0[others]) <= 0.1 * np.abs(sm0[others]))
    log("max logit without / with the norm: " +
        ", ".join(f"h{h}: {sm0[h]:.0f} / {sm1[h]:.1f}" for h in heads))
