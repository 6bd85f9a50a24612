"""GPU parity of the absorbed (inference) form (mla_absorbed) against the CPU oracle."""
import numpy as np
import pytest

import oracle
import synth
from tests._util import rel_err

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
F32_TOL = 1e-4
SMAX_TOL = 1e-3


@pytest.fixture(scope="module")
def lib(gpu_available):
    import mla_qk_clip_amd as m
    return m


def test_tiny_fp32_absorbed_matches_materialised_oracle(lib):
    """The tiny fp32 case as 64 queries over a 64-row cache: equals the
    training-form result (oracle) to 1e-4."""
    import mla_qk_clip_amd as m
    from tests._gpu import dev, dev_i32, host, lib_dims, log
    p, q4, cache, lens, g4 = synth.tiny_fp32_absorbed()
    log("tiny fp32 absorbed")
    out, ml = m.mla_absorbed(lib_dims(p.dims), dev(q4, False), dev(cache, False), dev_i32(lens),
                             dev(p.w_kv_b, False), dev(g4, False))
    ref, _, ref_sm = oracle.prefill(p.q, p.ckv, p.ks, p.w_kv_b, p.gate, p.cu_seqlens, p.dims)
    assert rel_err(host(out)[0], ref) <= F32_TOL
    assert np.all(np.abs(host(ml) - ref_sm) / np.abs(ref_sm) <= 1e-5)


@pytest.mark.parametrize("tq", [1, 3])
def test_fp32_decode_ragged(lib, tq):
    from tests._gpu import host, log, run_absorbed
    d = synth.decode_inputs(synth.TINY, [3, 64, 17, 100], cap=128, tq=tq, seed=31, bf16=False)
    log(f"fp32 absorbed tq={tq}")
    out, ml = run_absorbed(d)
    rows = [d.cache_rows(b) for b in range(d.batch)]
    ref, ref_sm = oracle.absorbed(d.q, rows, d.w_kv_b, d.gate, d.dims)
    assert rel_err(host(out), ref) <= F32_TOL
    assert np.all(np.abs(host(ml) - ref_sm) / np.abs(ref_sm) <= 1e-5)


@pytest.mark.parametrize("tq", [1, 2])
def test_bf16_decode_ragged_k3(lib, tq):
    """Lengths that are not multiples of the 32-row tile, shorter than a tile,
    and long enough to be split over several workgroups."""
    from tests._gpu import host, log, run_absorbed
    d = synth.decode_inputs(synth.K3, [5, 33, 1000, 4097, 31, 64], cap=4160, tq=tq, seed=32, bf16=True)
    log(f"bf16 absorbed ragged tq={tq}")
    out, ml = run_absorbed(d)
    rows = [d.cache_rows(b) for b in range(d.batch)]
    ref, ref_sm = oracle.absorbed(d.q, rows, d.w_kv_b, d.gate, d.dims)
    assert rel_err(host(out), ref) <= BF16_TOL
    assert np.all(np.abs(host(ml) - ref_sm) / np.abs(ref_sm) <= SMAX_TOL)


def test_bf16_decode_matches_prefill_last_row(lib):
    """Decode of the last position equals the training-form output of that row."""
    import torch
    from tests._gpu import dev, dev_i32, host, lib_dims, log, run_prefill
    import mla_qk_clip_amd as m
    p = synth.prefill_inputs(synth.K3, [300], seed=33, bf16=True)
    log("bf16 decode vs prefill last row")
    out_p, _, _ = run_prefill(p)
    cache = np.concatenate([p.ckv, p.ks], axis=1)[None]
    out_d, _ = m.mla_absorbed(lib_dims(p.dims), dev(p.q[None, -1:], True), dev(cache, True), dev_i32([300]),
                              dev(p.w_kv_b, True), dev(p.gate[None, -1:], True), out_dtype=torch.float32)
    torch.cuda.synchronize()
    a, b = host(out_d)[0, 0], host(out_p)[-1]
    assert rel_err(a, b) <= BF16_TOL


def test_bf16_k3_decode_workload(lib):
    """The absorbed-decode workload at full size: 64 sequences, cache rows of
    576 bf16 up to 32768 per sequence (NaN beyond each length), one query each.
    Outputs of 8 sequences against the oracle; the max logit over all 64."""
    from tests._gpu import host, log, run_absorbed
    d = synth.k3_decode()
    log(f"K3 decode workload: sum(lens)={int(d.lens.sum())}")
    out, ml = run_absorbed(d)
    assert bool(np.isfinite(host(out)).all())
    sample = [0, 9, 17, 26, 35, 44, 53, 63]
    rows = {b: d.cache_rows(b) for b in sample}
    log("oracle on sampled sequences")
    ref, _ = oracle.absorbed(d.q[sample], [rows[b] for b in sample], d.w_kv_b, d.gate[sample], d.dims)
    o = host(out)
    assert rel_err(o[sample], ref) <= BF16_TOL
    log("oracle max logit over all sequences")
    sm = np.full(d.dims.heads, -np.inf)
    w = d.w_kv_b.astype(np.float64)
    N, V = d.dims.nope_dim, d.dims.v_dim
    for b in range(d.batch):
        r = rows[b] if b in rows else d.cache_rows(b)
        qa = np.stack([oracle.mla_oracle.absorb_query(d.q[b, 0, h], w, d.dims, h) for h in range(d.dims.heads)])
        s = (r.astype(np.float64) @ qa.T) * d.dims.scale
        sm = np.maximum(sm, s.max(axis=0))
    assert np.all(np.abs(host(ml) - sm) / np.abs(sm) <= SMAX_TOL)
    del N, V


def test_bf16_decode_deterministic(lib):
    from tests._gpu import decode_cache_tensor, log, run_absorbed
    d = synth.decode_inputs(synth.K3, [2000, 777, 1], cap=2048, tq=1, seed=34, bf16=True)
    cache = decode_cache_tensor(d)
    log("decode determinism")
    o1, m1 = run_absorbed(d, cache=cache)
    o2, m2 = run_absorbed(d, cache=cache)
    assert bool((o1 == o2).all()) and bool((m1 == m2).all())
