"""GPU parity of the expanded-cache decode (mla_expanded) against the CPU oracle."""
import numpy as np
import pytest

import oracle
import synth
from tests._util import rel_err

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
SMAX_TOL = 1e-3


@pytest.fixture(scope="module")
def lib(gpu_available):
    import mla_qk_clip_amd as m
    return m


def _caches(dims, rows, cap):
    """Device k_cache [B, H, cap, N+S] and v_cache [B, H, cap, V] (bf16) from
    per-sequence (K [H, L, D], V [H, L, V]) rows; rows past each length hold NaN."""
    import torch
    from tests._gpu import dev
    B, H, D = len(rows), dims.heads, dims.nope_dim + dims.shared_dim
    kc = torch.full((B, H, cap, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    vc = torch.full((B, H, cap, dims.v_dim), float("nan"), dtype=torch.bfloat16, device="cuda")
    for b, (k, v) in enumerate(rows):
        L = k.shape[1]
        kc[b, :, :L] = dev(k, True)
        vc[b, :, :L] = dev(v, True)
    return kc, vc


def _run(dims, d, kc, vc, **kw):
    import torch
    import mla_qk_clip_amd as m
    from tests._gpu import dev, dev_i32, lib_dims
    out, ml = m.mla_expanded(lib_dims(dims), dev(d.q, True), kc, vc, dev_i32(d.lens),
                             None if d.gate is None else dev(d.gate, True), **kw)
    torch.cuda.synchronize()
    return out, ml


@pytest.mark.parametrize("tq", [1, 3])
@pytest.mark.parametrize("out_f32", [False, True])
def test_bf16_expanded_ragged(lib, tq, out_f32):
    """Lengths around the 2048-row split (one row over, exactly one split,
    three splits with a ragged tail), shorter than an 8-row pass, and a query
    that sees a single row (lens = tq)."""
    import torch
    from tests._gpu import host, log
    dims = synth.Dims(8, 512, 64, 128, 128)
    lens = [3, 2049, 4100, 40, 2048]
    d = synth.decode_inputs(dims, lens, cap=4160, tq=tq, seed=41, bf16=True)
    rows = [synth.expanded_rows(dims, L, seed=41, b=b) for b, L in enumerate(lens)]
    log(f"bf16 expanded ragged tq={tq} out_f32={out_f32}")
    kc, vc = _caches(dims, rows, 4160)
    out, ml = _run(dims, d, kc, vc, out_dtype=torch.float32 if out_f32 else None)
    ref, ref_sm = oracle.expanded(d.q, [r[0] for r in rows], [r[1] for r in rows], d.gate, dims)
    assert out.dtype == (torch.float32 if out_f32 else torch.bfloat16)
    assert rel_err(host(out), ref) <= BF16_TOL
    assert np.all(np.abs(host(ml) - ref_sm) / np.abs(ref_sm) <= SMAX_TOL)


def test_bf16_expanded_equals_latent_decode(lib):
    """Per-head K/V formed from latent rows (then rounded to bf16) give the
    absorbed form's result on those latent rows (oracle), up to the rounding
    of the expanded rows."""
    from tests._gpu import host, log
    dims = synth.Dims(4, 512, 64, 128, 128)
    lens = [100, 2100, 7]
    d = synth.decode_inputs(dims, lens, cap=2176, tq=2, seed=42, bf16=True)
    lat = [d.cache_rows(b) for b in range(d.batch)]
    k_rows, v_rows = oracle.expanded_cache(lat, d.w_kv_b, dims)
    rows = [(synth.round_bf16(k.astype(np.float32)), synth.round_bf16(v.astype(np.float32)))
            for k, v in zip(k_rows, v_rows)]
    log("bf16 expanded vs latent rows")
    kc, vc = _caches(dims, rows, 2176)
    out, ml = _run(dims, d, kc, vc)
    ref, ref_sm = oracle.absorbed(d.q, lat, d.w_kv_b, d.gate, dims)
    assert rel_err(host(out), ref) <= BF16_TOL
    assert np.all(np.abs(host(ml) - ref_sm) / np.abs(ref_sm) <= 5e-3)


def test_bf16_expanded_single_row_no_gate_and_accumulate(lib):
    """lens = tq = 1 (one visible row: out = its V row), no gate; accumulate
    keeps a larger prior maximum and replaces a smaller one."""
    import torch
    from tests._gpu import host, log
    dims = synth.Dims(4, 512, 64, 128, 128)
    lens = [1, 9]
    d = synth.decode_inputs(dims, lens, cap=16, tq=1, seed=43, bf16=True, gate=False)
    rows = [synth.expanded_rows(dims, L, seed=43, b=b) for b, L in enumerate(lens)]
    log("bf16 expanded single row / accumulate")
    kc, vc = _caches(dims, rows, 16)
    prior = torch.tensor([1e3, -1e3, 1e3, -1e3], dtype=torch.float32, device="cuda")
    out, ml = _run(dims, d, kc, vc, out_dtype=torch.float32, max_logit=prior, accumulate=True)
    ref, ref_sm = oracle.expanded(d.q, [r[0] for r in rows], [r[1] for r in rows], None, dims)
    assert rel_err(host(out), ref) <= BF16_TOL
    assert np.allclose(host(out)[0, 0], rows[0][1][:, 0].reshape(-1), rtol=0, atol=0)
    got = host(ml)
    assert got[0] == 1e3 and got[2] == 1e3
    assert abs(got[1] - ref_sm[1]) <= SMAX_TOL * abs(ref_sm[1]) and abs(got[3] - ref_sm[3]) <= SMAX_TOL * abs(ref_sm[3])


def test_bf16_expanded_deterministic(lib):
    import torch
    from tests._gpu import log
    dims = synth.Dims(8, 512, 64, 128, 128)
    lens = [3000, 517]
    d = synth.decode_inputs(dims, lens, cap=3008, tq=1, seed=44, bf16=True)
    rows = [synth.expanded_rows(dims, L, seed=44, b=b) for b, L in enumerate(lens)]
    log("bf16 expanded determinism")
    kc, vc = _caches(dims, rows, 3008)
    a, ma = _run(dims, d, kc, vc)
    b, mb = _run(dims, d, kc, vc)
    assert torch.equal(a, b) and torch.equal(ma, mb)


def test_bf16_expanded_k3_decode_workload_sampled(lib):
    """The Kimi K3 decode workload (64 sequences, lens ~ U[1024, 32768], cap
    32768, 96 heads, gate on) with a per-head cache of 129 GB: sampled
    (sequence, head) outputs against the oracle, and every head's max logit.
    Each head h has one planted row in sequence h % 64 equal to its query, so
    its maximum (|q|^2 / sqrt(192) >= 7.9 against about 5.3 for the random rows)
    sits in a known sequence, which the oracle then covers exactly."""
    import torch
    import mla_qk_clip_amd as m
    from tests._gpu import dev, dev_i32, host, lib_dims, log
    d = synth.k3_decode()
    dims = d.dims
    B, H, cap, D, V = d.batch, dims.heads, d.cap, dims.nope_dim + dims.shared_dim, dims.v_dim
    lens = d.lens.astype(np.int64)
    log(f"K3 expanded decode: B={B} cap={cap} sum(lens)={int(lens.sum())}")
    g = torch.Generator(device="cuda")
    g.manual_seed(45)
    kc = torch.randn((B, H, cap, D), generator=g, dtype=torch.bfloat16, device="cuda")
    vc = torch.randn((B, H, cap, V), generator=g, dtype=torch.bfloat16, device="cuda")
    for b in range(B):
        kc[b, :, int(lens[b]):] = float("nan")
        vc[b, :, int(lens[b]):] = float("nan")
    q = dev(d.q, True)
    plant = {h: (h % B, int(lens[h % B]) // 2) for h in range(H)}
    for h, (b, j) in plant.items():
        kc[b, h, j] = q[b, 0, h]
    torch.cuda.synchronize()
    log("caches filled")
    out, ml = m.mla_expanded(lib_dims(dims), q, kc, vc, dev_i32(d.lens), dev(d.gate, True))
    torch.cuda.synchronize()
    log("expanded decode done")
    got_out, got_ml = host(out), host(ml)
    # every head's max logit: the oracle over the sequence that holds the planted row
    for h, (b, j) in plant.items():
        L = int(lens[b])
        k = kc[b, h:h + 1, :L].float().cpu().numpy()
        v = vc[b, h:h + 1, :L].float().cpu().numpy()
        _, sm = oracle.expanded(d.q[b:b + 1, :, h:h + 1], [k], [v], None, synth.Dims(1, 512, 64, 128, 128))
        assert abs(got_ml[h] - sm[0]) <= SMAX_TOL * abs(sm[0]), (h, got_ml[h], sm[0])
    # sampled outputs from sequences without a planted row for that head
    rng = np.random.default_rng(46)
    for _ in range(16):
        h = int(rng.integers(H))
        b = int(rng.integers(B))
        if b == plant[h][0]:
            b = (b + 1) % B
        L = int(lens[b])
        k = kc[b, h:h + 1, :L].float().cpu().numpy()
        v = vc[b, h:h + 1, :L].float().cpu().numpy()
        ref, _ = oracle.expanded(d.q[b:b + 1, :, h:h + 1], [k], [v], d.gate[b:b + 1, :, h * V:(h + 1) * V],
                                 synth.Dims(1, 512, 64, 128, 128))
        assert rel_err(got_out[b, 0, h * V:(h + 1) * V], ref[0, 0]) <= BF16_TOL, (b, h)
    del kc, vc
    torch.cuda.empty_cache()
