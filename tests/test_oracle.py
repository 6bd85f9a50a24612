"""Pins for the CPU oracle: each test checks it against something other than
itself (closed forms, a library routine, brute force, invariants, the pages'
printed numbers), chosen so that a dropped term, a wrong sign or index, or a
transposed operand in the oracle fails at least one of them.
"""
import math
import os

import numpy as np
import pytest

import oracle
import synth
from tests._util import rel_err

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                vals[k] = int(v)
    return vals


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _id_weights(dims, uv_of_head, uk_of_head=None):
    """kv_b_proj.weight [H*(N+V), R] built from per-head blocks (rows = output features)."""
    H, R, N, V = dims.heads, dims.kv_rank, dims.nope_dim, dims.v_dim
    w = np.zeros((H * (N + V), R))
    for h in range(H):
        w[h * (N + V):h * (N + V) + N] = np.eye(N, R) if uk_of_head is None else uk_of_head(h)
        w[h * (N + V) + N:(h + 1) * (N + V)] = uv_of_head(h)
    return w


# ---------------------------------------------------------------------------
# generator and rounding
# ---------------------------------------------------------------------------


def test_generator_is_deterministic():
    a = synth.prefill_inputs(synth.TINY, [5, 7], seed=3, bf16=True)
    b = synth.prefill_inputs(synth.TINY, [5, 7], seed=3, bf16=True)
    c = synth.prefill_inputs(synth.TINY, [5, 7], seed=4, bf16=True)
    for x, y in [(a.q, b.q), (a.ckv, b.ckv), (a.w_kv_b, b.w_kv_b), (a.gate, b.gate)]:
        assert np.array_equal(x, y)
    assert not np.array_equal(a.q, c.q)
    assert list(a.cu_seqlens) == [0, 5, 12]
    d = synth.decode_inputs(synth.TINY, [3, 9], cap=16, tq=1, seed=5, bf16=True)
    assert np.array_equal(d.cache_rows(1), d.cache_rows(1))
    assert d.cache_rows(0).shape == (3, 48)


def test_bf16_rounding_two_implementations_agree():
    # synth rounds float32 with integer bit arithmetic; the oracle rounds float64
    # with frexp/rint. Both are round-to-nearest-even to 8 significant bits.
    one = 1.0
    assert oracle.round_to(one + 2.0 ** -8, "bf16") == 1.0                       # tie -> even
    assert oracle.round_to(one + 3 * 2.0 ** -8, "bf16") == one + 2.0 ** -6       # tie -> even
    assert oracle.round_to(one + 2.0 ** -8 + 2.0 ** -20, "bf16") == one + 2.0 ** -7
    assert synth.round_bf16(np.float32([one + 2.0 ** -8]))[0] == 1.0
    assert synth.round_bf16(np.float32([one + 3 * 2.0 ** -8]))[0] == one + 2.0 ** -6
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 37
    assert np.array_equal(synth.round_bf16(x).astype(np.float64), oracle.round_to(x.astype(np.float64), "bf16"))
    bits = synth.bf16_bits(synth.round_bf16(x))
    assert np.array_equal(synth.from_bf16_bits(bits), synth.round_bf16(x))


def test_bf16_rounding_over_the_whole_float32_range():
    """Both roundings over every binade of float32, its subnormals and the
    overflow threshold: bf16 keeps fp32's exponent range, so values below
    2^-126 round to multiples of 2^-133 and values at or past the midpoint
    between the largest finite bf16 value and 2^128 become infinite."""
    rng = np.random.default_rng(1)
    # random bit patterns cover every exponent (normal and subnormal) and sign
    u = rng.integers(0, 2 ** 32, size=400000, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    x = x[np.isfinite(x)]
    a = synth.round_bf16(x).astype(np.float64)
    b = oracle.round_to(x.astype(np.float64), "bf16")
    assert np.array_equal(a, b)
    bmax = (2.0 - 2.0 ** -7) * 2.0 ** 127
    edge = np.array([bmax, (2.0 - 2.0 ** -8) * 2.0 ** 127, np.nextafter(np.float32((2.0 - 2.0 ** -8) * 2.0 ** 127),
                     np.float32(0)), 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -134, 2.0 ** -126 - 2.0 ** -140,
                     np.float32(3.4e38)], dtype=np.float32)
    assert np.array_equal(synth.round_bf16(edge).astype(np.float64), oracle.round_to(edge.astype(np.float64), "bf16"))
    assert oracle.round_to(bmax, "bf16") == bmax
    assert oracle.round_to((2.0 - 2.0 ** -8) * 2.0 ** 127, "bf16") == np.inf     # tie: to even (overflow)
    assert oracle.round_to(-(2.0 - 2.0 ** -8) * 2.0 ** 127, "bf16") == -np.inf
    assert oracle.round_to(2.0 ** -134, "bf16") == 0.0                             # half the smallest step: to even
    assert oracle.round_to(3 * 2.0 ** -134, "bf16") == 2.0 ** -132                 # 1.5 steps: to even (2 steps)
    assert oracle.round_to(2.0 ** -126 - 2.0 ** -140, "bf16") == 2.0 ** -126
    assert np.isnan(oracle.round_to(np.nan, "bf16"))


# ---------------------------------------------------------------------------
# the pages' printed numbers
# ---------------------------------------------------------------------------


def test_layer_parameter_accounting_matches_page():
    """The weight layouts used here (q_b_proj [H*D, q_in], kv_b_proj [H*(N+V), R],
    a joint down-projection of width R + S) reproduce the page's exact counts."""
    g = _golden("k3_mla_parameters.txt")
    d = synth.K3
    hidden, q_in = 7168, synth.K3_Q_LORA_RANK
    D = d.nope_dim + d.shared_dim
    w_dq = hidden * q_in
    q_norm = q_in
    w_q_b = (d.heads * D) * q_in
    w_dkv = hidden * (d.kv_rank + d.shared_dim)
    kv_norm = d.kv_rank
    w_kv_b = (d.heads * (d.nope_dim + d.v_dim)) * d.kv_rank
    w_g = hidden * d.heads * d.v_dim
    w_o = d.heads * d.v_dim * hidden
    assert w_dq + q_norm + w_q_b == g["query_heads"]
    assert w_dkv + kv_norm + w_kv_b == g["key_and_value_heads"]
    assert w_g == g["output_gate_projection"]
    assert w_o == g["output_projection"]
    total = w_dq + q_norm + w_q_b + w_dkv + kv_norm + w_kv_b + w_g + w_o
    assert total == g["per_instance_total"]
    assert total * 24 == g["all_24_layers"]


def test_cache_row_width_matches_page():
    g = _golden("k3_cache_widths.txt")
    d = synth.K3
    assert 2 * d.heads * d.v_dim == g["classic_values"]
    assert d.kv_rank == g["mla_latent"] and d.shared_dim == g["mla_shared"]
    assert round(g["classic_values"] / (d.kv_rank + d.shared_dim)) == g["ratio_rounded"]


# ---------------------------------------------------------------------------
# materialised (training) form
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("gate", [True, False])
def test_blocked_oracle_equals_brute_force(gate):
    p = synth.prefill_inputs(synth.TINY, [23, 1, 0, 40], seed=11, bf16=False, gate=gate)
    out, lse, sm = oracle.prefill(p.q, p.ckv, p.ks, p.w_kv_b, p.gate, p.cu_seqlens, p.dims, block=7)
    out2, probs, sm2 = oracle.dense_prefill(p.q, p.ckv, p.ks, p.w_kv_b, p.gate, p.cu_seqlens, p.dims)
    assert rel_err(out, out2) < 1e-12
    assert np.allclose(sm, sm2, rtol=1e-13, atol=0)
    # lse brackets the row maximum: max_s S <= lse <= max_s S + log(#visible)
    assert np.all(np.isfinite(lse))


def test_softmax_rows_sum_to_one_and_masked_weights_are_zero():
    p = synth.prefill_inputs(synth.TINY, [9, 14], seed=2, bf16=False)
    _, probs, _ = oracle.dense_prefill(p.q, p.ckv, p.ks, p.w_kv_b, p.gate, p.cu_seqlens, p.dims)
    assert np.allclose(probs.sum(axis=-1), 1.0, atol=1e-14)
    n = int(p.cu_seqlens[-1])
    seq = np.repeat([0, 1], [9, 14])
    pos = np.arange(n)
    forbidden = (seq[:, None] != seq[None, :]) | (pos[None, :] > pos[:, None])
    assert np.all(probs[:, forbidden] == 0.0)
    assert np.all(probs[:, ~forbidden] > 0.0)


def test_single_token_returns_gated_value_row():
    """T = 1: the only weight is 1, so o = sigma(g) . V_0 with V_0 = c_0 W_UV_h.
    With W_UV_h = (h+1) I (and random W_UK_h) this is (h+1) sigma(g) c_0."""
    dims = oracle.Dims(3, 8, 4, 8, 8)
    rng = np.random.default_rng(0)
    w = _id_weights(dims, lambda h: (h + 1) * np.eye(8), lambda h: rng.standard_normal((8, 8)))
    q, ckv, ks, g = _rand(rng, 1, 3, 12), _rand(rng, 1, 8), _rand(rng, 1, 4), _rand(rng, 1, 24)
    out, lse, sm = oracle.prefill(q, ckv, ks, w, g, [0, 1], dims)
    expect = np.concatenate([(h + 1) * ckv[0] for h in range(3)]) / (1 + np.exp(-g[0]))
    assert rel_err(out[0], expect) < 1e-14
    assert np.allclose(lse[:, 0], sm)          # one visible key: lse = its logit


def test_zero_query_gives_prefix_mean_per_sequence():
    """q = 0: every visible logit is 0, A_{t,s} = 1/(t+1), so O~_t is the running
    mean of V over its own sequence."""
    dims = oracle.Dims(2, 6, 3, 6, 6)
    rng = np.random.default_rng(1)
    w = _id_weights(dims, lambda h: (2 * h - 1.5) * np.eye(6), lambda h: rng.standard_normal((6, 6)))
    lens = [5, 8]
    n = sum(lens)
    ckv, ks = _rand(rng, n, 6), _rand(rng, n, 3)
    q = np.zeros((n, 2, 9))
    out, lse, sm = oracle.prefill(q, ckv, ks, w, None, [0, 5, 13], dims)
    expect = np.zeros((n, 12))
    for a, b in [(0, 5), (5, 13)]:
        cm = np.cumsum(ckv[a:b], axis=0) / np.arange(1, b - a + 1)[:, None]
        for h in range(2):
            expect[a:b, h * 6:(h + 1) * 6] = (2 * h - 1.5) * cm
    assert rel_err(out, expect) < 1e-14
    assert np.all(sm == 0.0)
    pos = np.array([0, 1, 2, 3, 4, 0, 1, 2, 3, 4, 5, 6, 7])
    assert np.allclose(lse, np.log(pos + 1)[None], atol=1e-15)


def test_gate_zero_halves_and_saturated_gate_selects_heads():
    p = synth.prefill_inputs(synth.TINY, [17], seed=5, bf16=False)
    ungated, _, _ = oracle.prefill(p.q, p.ckv, p.ks, p.w_kv_b, None, p.cu_seqlens, p.dims)
    half, _, _ = oracle.prefill(p.q, p.ckv, p.ks, p.w_kv_b, np.zeros_like(p.gate), p.cu_seqlens, p.dims)
    assert rel_err(half, ungated / 2) < 1e-15
    V = p.dims.v_dim
    g = np.full_like(p.gate, -800.0)
    g[:, 2 * V:3 * V] = 800.0                  # open head 2 only
    sel, _, _ = oracle.prefill(p.q, p.ckv, p.ks, p.w_kv_b, g, p.cu_seqlens, p.dims)
    assert np.array_equal(sel[:, 2 * V:3 * V], ungated[:, 2 * V:3 * V])
    assert np.all(sel[:, :2 * V] == 0) and np.all(sel[:, 3 * V:] == 0)


def test_matches_torch_causal_sdpa_in_identity_special_case():
    """R = N, W_UK_h = I, W_UV_h = a permutation P_h: then K_h = [c, k^S] and
    V_h = c P_h^T, so each head is textbook causal scaled-dot-product attention
    with the default scale 1/sqrt(q width) = 1/sqrt(N+S)."""
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    H, N, S = 3, 16, 8
    dims = oracle.Dims(H, N, S, N, N)
    rng = np.random.default_rng(7)
    perms = [rng.permutation(N) for _ in range(H)]
    w = _id_weights(dims, lambda h: np.eye(N)[perms[h]])
    T = 37
    q, ckv, ks = _rand(rng, T, H, N + S), _rand(rng, T, N), _rand(rng, T, S)
    out, _, _ = oracle.prefill(q, ckv, ks, w, None, [0, T], dims, block=8)
    for h in range(H):
        qt = torch.from_numpy(q[:, h, :])[None, None]
        kt = torch.from_numpy(np.concatenate([ckv, ks], axis=1))[None, None]
        vt = torch.from_numpy(ckv[:, perms[h]])[None, None]
        ref = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True)[0, 0].numpy()
        assert rel_err(out[:, h * N:(h + 1) * N], ref) < 1e-12


def test_max_logit_closed_form_respects_causality():
    """q_t = (T-1-t) e_1, c_s = s e_1, k^S = 0, W_UK = I: logit(t, s) =
    (T-1-t) s / sqrt(D) for s <= t, largest at t = floor((T-1)/2) with value
    t (T-1-t) / sqrt(D). Without the mask it would be (T-1)^2 / sqrt(D)."""
    dims = oracle.Dims(1, 4, 2, 4, 4)
    D = 6
    lens = [64, 9]
    qs, cs = [], []
    for T in lens:
        q = np.zeros((T, 1, D))
        q[:, 0, 0] = np.arange(T - 1, -1, -1)
        c = np.zeros((T, 4))
        c[:, 0] = np.arange(T)
        qs.append(q)
        cs.append(c)
    q = np.concatenate(qs)
    c = np.concatenate(cs)
    ks = np.zeros((sum(lens), 2))
    w = _id_weights(dims, lambda h: np.eye(4))
    _, _, sm = oracle.prefill(q, c, ks, w, None, [0, 64, 73], dims, block=16)
    assert sm[0] == pytest.approx(31 * 32 / math.sqrt(D), rel=1e-15)
    assert oracle.max_logit_head(q, c, ks, w, [0, 64, 73], dims, 0) == pytest.approx(31 * 32 / math.sqrt(D), rel=1e-15)
    _, _, sm2 = oracle.dense_prefill(q, c, ks, w, None, [0, 64, 73], dims)
    assert sm2[0] == pytest.approx(31 * 32 / math.sqrt(D), rel=1e-15)


def test_lse_brackets_row_max_and_rows_are_independent():
    p = synth.prefill_inputs(synth.TINY, [30], seed=9, bf16=False)
    out, lse, sm = oracle.prefill(p.q, p.ckv, p.ks, p.w_kv_b, p.gate, p.cu_seqlens, p.dims, block=4)
    for h in range(p.dims.heads):
        rows = [0, 7, 29]
        o, l = oracle.prefill_rows(p.q, p.ckv, p.ks, p.w_kv_b, p.gate, p.cu_seqlens, p.dims, h, rows)
        V = p.dims.v_dim
        assert rel_err(o, out[rows, h * V:(h + 1) * V]) < 1e-13
        assert np.allclose(l, lse[h, rows], rtol=1e-14)
    assert np.all(lse.max(axis=1) >= sm - 1e-12)
    assert np.all(lse[:, 0] <= sm + 1e-12)   # row 0 has a single key


# ---------------------------------------------------------------------------
# absorbed (inference) form
# ---------------------------------------------------------------------------


def test_absorbed_equals_materialised_on_tiny_fp32_workload():
    p, q4, cache, lens, g4 = synth.tiny_fp32_absorbed()
    ref, _, sm_ref = oracle.prefill(p.q, p.ckv, p.ks, p.w_kv_b, p.gate, p.cu_seqlens, p.dims)
    out, sm = oracle.absorbed(q4, [cache[0]], p.w_kv_b, g4, p.dims)
    assert rel_err(out[0], ref) < 1e-10
    assert np.allclose(sm, sm_ref, rtol=1e-12)


@pytest.mark.parametrize("tq", [1, 3])
def test_absorbed_decode_is_last_rows_of_prefill(tq):
    dims = synth.TINY
    p = synth.prefill_inputs(dims, [21, 40], seed=4, bf16=True)
    ref, _, _ = oracle.prefill(p.q, p.ckv, p.ks, p.w_kv_b, p.gate, p.cu_seqlens, p.dims)
    rows = [np.concatenate([p.ckv[a:b], p.ks[a:b]], axis=1) for a, b in [(0, 21), (21, 61)]]
    q = np.stack([p.q[21 - tq:21], p.q[61 - tq:61]])
    g = np.stack([p.gate[21 - tq:21], p.gate[61 - tq:61]])
    out, sm = oracle.absorbed(q, rows, p.w_kv_b, g, dims)
    assert rel_err(out[0], ref[21 - tq:21]) < 1e-10
    assert rel_err(out[1], ref[61 - tq:61]) < 1e-10
    sm_rows = oracle.absorbed_rows_selected(q, rows, p.w_kv_b, g, dims, [0, 1])[1]
    assert np.array_equal(sm_rows, sm)


def test_absorbed_max_logit_matches_materialised_last_rows():
    dims = synth.TINY
    p = synth.prefill_inputs(dims, [33], seed=8, bf16=True)
    tq = 5
    rows = [np.concatenate([p.ckv, p.ks], axis=1)]
    _, sm = oracle.absorbed(p.q[None, 33 - tq:], rows, p.w_kv_b, None, dims)
    # the same logits from the materialised side: K_h = [K^C_h, k^S], scaled dot
    for h in range(dims.heads):
        kc, _ = oracle.expand_latent(p.ckv, p.w_kv_b, dims, h)
        K = np.concatenate([kc, p.ks], axis=1)
        best = -np.inf
        for t in range(33 - tq, 33):
            best = max(best, float((K[:t + 1] @ p.q[t, h].astype(np.float64)).max()) * oracle.mla_oracle.scale_of(dims))
        assert sm[h] == pytest.approx(best, rel=1e-12)


@pytest.mark.parametrize("tq", [1, 4])
def test_absorbed_max_logit_alone_matches_materialised_keys(tq):
    """``absorbed_max_logit`` (no softmax) against the materialised side: the
    key K_h = [c^KV W_UK_h, k^S] of every visible row scored with q directly,
    on ragged sequences of several lengths; and against ``absorbed``'s own
    maximum on the same inputs."""
    dims = synth.TINY
    d = synth.decode_inputs(dims, [9, 1 + tq, 30], cap=32, tq=tq, seed=12, bf16=True)
    rows = [d.cache_rows(b) for b in range(d.batch)]
    sm = oracle.absorbed_max_logit(d.q, rows, d.w_kv_b, dims)
    _, sm_full = oracle.absorbed(d.q, rows, d.w_kv_b, d.gate, dims)
    assert np.allclose(sm, sm_full, rtol=1e-12, atol=0)
    R = dims.kv_rank
    scale = 1.0 / math.sqrt(dims.nope_dim + dims.shared_dim)
    for h in range(dims.heads):
        best = -np.inf
        for b, r in enumerate(rows):
            kc, _ = oracle.expand_latent(r[:, :R], d.w_kv_b, dims, h)
            K = np.concatenate([kc, r[:, R:].astype(np.float64)], axis=1)
            L = r.shape[0]
            for i in range(tq):
                vis = L - tq + i + 1
                best = max(best, float((K[:vis] @ d.q[b, i, h].astype(np.float64)).max()) * scale)
        assert sm[h] == pytest.approx(best, rel=1e-12)
    # a row planted late in one sequence and visible only to the last query
    rows2 = [r.copy() for r in rows]
    rows2[2][-1] = rows2[2][-1] * 50.0
    sm2 = oracle.absorbed_max_logit(d.q, rows2, d.w_kv_b, dims)
    assert np.all(sm2 >= sm - 1e-12) and np.any(sm2 > 10 * np.abs(sm))


# ---------------------------------------------------------------------------
# Expanded-cache decode (per-head K and V rows)
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("tq", [1, 3])
def test_expanded_equals_absorbed_on_latent_derived_cache(tq):
    """Per-head K/V built from latent rows give the absorbed form's result
    (associativity of the [MLA] equations), outputs and max logits."""
    dims = synth.TINY
    rng = np.random.default_rng(31)
    lens = [7, 19, 12]
    rows = [rng.standard_normal((L, dims.kv_rank + dims.shared_dim)) for L in lens]
    w = rng.standard_normal((dims.heads * (dims.nope_dim + dims.v_dim), dims.kv_rank)) / math.sqrt(dims.kv_rank)
    D = dims.nope_dim + dims.shared_dim
    q = rng.standard_normal((len(lens), tq, dims.heads, D))
    g = rng.standard_normal((len(lens), tq, dims.heads * dims.v_dim))
    ref, sm_ref = oracle.absorbed(q, rows, w, g, dims)
    k_rows, v_rows = oracle.expanded_cache(rows, w, dims)
    assert k_rows[1].shape == (dims.heads, 19, D) and v_rows[1].shape == (dims.heads, 19, dims.v_dim)
    out, sm = oracle.expanded(q, k_rows, v_rows, g, dims)
    assert rel_err(out, ref) < 1e-10
    assert np.allclose(sm, sm_ref, rtol=1e-12)


def test_expanded_with_all_positions_queried_is_dense_causal_attention():
    """Tq = L: every position of the sequence is a query, so the decode form is
    the brute-force masked softmax of the training form."""
    dims = synth.TINY
    p = synth.prefill_inputs(dims, [23], seed=12, bf16=False)
    ref, _, sm_ref = oracle.dense_prefill(p.q, p.ckv, p.ks, p.w_kv_b, p.gate, p.cu_seqlens, dims)
    rows = [np.concatenate([p.ckv, p.ks], axis=1)]
    k_rows, v_rows = oracle.expanded_cache(rows, p.w_kv_b, dims)
    out, sm = oracle.expanded(p.q[None], k_rows, v_rows, p.gate[None], dims)
    assert rel_err(out[0], ref) < 1e-10
    assert np.allclose(sm, sm_ref, rtol=1e-12)


def test_expanded_zero_query_gives_prefix_mean_of_values():
    """q = 0: every visible score is 0, so query i returns the mean of the
    first L - Tq + i + 1 value rows (times the gate)."""
    dims = synth.TINY
    rng = np.random.default_rng(5)
    L, tq = 11, 4
    D = dims.nope_dim + dims.shared_dim
    K = rng.standard_normal((dims.heads, L, D))
    Vv = rng.standard_normal((dims.heads, L, dims.v_dim))
    g = rng.standard_normal((1, tq, dims.heads * dims.v_dim))
    out, sm = oracle.expanded(np.zeros((1, tq, dims.heads, D)), [K], [Vv], g, dims)
    sig = 1.0 / (1.0 + np.exp(-g))
    for i in range(tq):
        vis = L - tq + i + 1
        want = Vv[:, :vis].mean(axis=1).reshape(-1)
        assert np.allclose(out[0, i], sig[0, i] * want, rtol=0, atol=1e-13)
    assert np.all(sm == 0.0)


def test_expanded_single_visible_row_returns_gated_value_row():
    dims = synth.TINY
    rng = np.random.default_rng(6)
    D = dims.nope_dim + dims.shared_dim
    K = rng.standard_normal((dims.heads, 1, D))
    Vv = rng.standard_normal((dims.heads, 1, dims.v_dim))
    q = rng.standard_normal((1, 1, dims.heads, D))
    g = rng.standard_normal((1, 1, dims.heads * dims.v_dim))
    out, sm = oracle.expanded(q, [K], [Vv], g, dims)
    assert np.allclose(out[0, 0], Vv[:, 0].reshape(-1) / (1.0 + np.exp(-g[0, 0])), rtol=1e-14, atol=0)
    want = np.array([K[h, 0] @ q[0, 0, h] for h in range(dims.heads)]) / math.sqrt(D)
    assert np.allclose(sm, want, rtol=1e-14, atol=0)


# ---------------------------------------------------------------------------
# Backward of the prefill
# ---------------------------------------------------------------------------


def test_prefill_backward_matches_central_differences():
    """Every gradient against central differences of the forward oracle along
    random directions: d/de <dO, out(x + e v)> = <grad_x, v> for x = q, c^KV,
    k^S, kv_b_proj.weight and the gate logits (two sequences, causal)."""
    dims = synth.TINY
    p = synth.prefill_inputs(dims, [6, 9], seed=61, bf16=False)
    rng = np.random.default_rng(62)
    dout = rng.standard_normal((p.ntok, dims.heads * dims.v_dim))
    grads = oracle.prefill_backward(p.q, p.ckv, p.ks, p.w_kv_b, p.gate, p.cu_seqlens, dims, dout)
    base = dict(q=p.q.astype(np.float64), ckv=p.ckv.astype(np.float64), ks=p.ks.astype(np.float64),
                w=p.w_kv_b.astype(np.float64), g=p.gate.astype(np.float64))

    def loss(**over):
        a = dict(base)
        a.update(over)
        out = oracle.prefill(a["q"], a["ckv"], a["ks"], a["w"], a["g"], p.cu_seqlens, dims)[0]
        return float(np.sum(out * dout))
    eps = 1e-5
    for name, g in zip(["q", "ckv", "ks", "w", "g"], grads):
        for _ in range(2):
            v = rng.standard_normal(base[name].shape)
            fd = (loss(**{name: base[name] + eps * v}) - loss(**{name: base[name] - eps * v})) / (2 * eps)
            assert abs(fd - float(np.sum(g * v))) <= 1e-7 * max(1.0, abs(fd)), name


def test_prefill_backward_value_gradient_closed_form_for_zero_query():
    """q = 0: the softmax rows are uniform over the causal prefix, so the value
    gradient at row s is sum over t >= s of dO~_t / (t + 1), dq's key part is
    the only q gradient path, and without a gate dO~ = dO."""
    dims = synth.TINY
    p = synth.prefill_inputs(dims, [7], seed=63, bf16=False, gate=False)
    rng = np.random.default_rng(64)
    dout = rng.standard_normal((7, dims.heads * dims.v_dim))
    q0 = np.zeros_like(p.q)
    _, dckv, dks, dw, dg = oracle.prefill_backward(q0, p.ckv, p.ks, p.w_kv_b, None, p.cu_seqlens, dims, dout)
    assert dg is None
    N, V, R = dims.nope_dim, dims.v_dim, dims.kv_rank
    # with q = 0 the keys get no gradient: dK = scale dS^T Q = 0, so dks = 0 and W_UK gets none
    assert np.all(dks == 0.0)
    for h in range(dims.heads):
        assert np.all(dw[h * (N + V):h * (N + V) + N] == 0.0)
        dV = np.zeros((7, V))
        for s in range(7):
            for t in range(s, 7):
                dV[s] += dout[t, h * V:(h + 1) * V] / (t + 1)
        want = dV.T @ p.ckv.astype(np.float64)      # d W_UV_h (rows)
        assert np.allclose(dw[h * (N + V) + N:(h + 1) * (N + V)], want, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# The whole layer (projections, RMSNorms, attention, output projection)
# ---------------------------------------------------------------------------


def test_rms_norm_closed_forms():
    w = np.array([1.0, 2.0, -0.5])
    # a constant row c: mean(x^2) = c^2, so x / sqrt(c^2 + eps) = c / sqrt(c^2 + eps)
    c, eps = 3.0, 1e-6
    got = oracle.rms_norm(np.full((1, 3), c), w, eps)
    assert np.allclose(got, w * c / math.sqrt(c * c + eps), rtol=1e-15, atol=0)
    # [3, 4, 0]: mean of squares 25/3
    got = oracle.rms_norm(np.array([[3.0, 4.0, 0.0]]), w, 0.0)
    assert np.allclose(got, np.array([3.0, 8.0, 0.0]) / math.sqrt(25.0 / 3.0), rtol=1e-15, atol=0)
    # scale invariance (eps = 0) and eps only matters near zero
    x = np.random.default_rng(1).standard_normal((4, 3))
    assert np.allclose(oracle.rms_norm(7.5 * x, w, 0.0), oracle.rms_norm(x, w, 0.0), rtol=1e-13, atol=0)


def test_linear_matches_brute_force_sums():
    rng = np.random.default_rng(2)
    x, w = rng.standard_normal((3, 5)), rng.standard_normal((4, 5))
    want = np.array([[sum(x[i, k] * w[j, k] for k in range(5)) for j in range(4)] for i in range(3)])
    assert np.allclose(oracle.linear(x, w), want, rtol=1e-14, atol=1e-15)


def _tiny_layer(seed=3, seqlens=(9, 14)):
    return synth.layer_inputs(synth.TINY, 40, 24, list(seqlens), seed, bf16=False)


def _layer(L, eps=1e-6, **over):
    a = dict(x=L.x, w_dq=L.w_dq, g_q=L.g_q, w_uq=L.w_uq, w_kv_a=L.w_kv_a, g_kv=L.g_kv, w_kv_b=L.w_kv_b, w_g=L.w_g,
             w_o=L.w_o)
    a.update(over)
    return oracle.layer_forward(a["x"], a["w_dq"], a["g_q"], a["w_uq"], a["w_kv_a"], a["g_kv"], a["w_kv_b"], a["w_g"],
                                a["w_o"], L.cu_seqlens, L.dims, eps, round_bf16=False)


def test_layer_norms_follow_the_down_projections():
    """The RMSNorms sit on c^Q and on c^KV only: scaling W_DQ, or the c^KV rows
    of W_DKV, leaves Delta unchanged (eps = 0); scaling the k^S rows does not."""
    L = _tiny_layer()
    R = L.dims.kv_rank
    ref, sm = _layer(L, eps=0.0)
    wkv = L.w_kv_a.copy()
    wkv[:R] *= 8.0   # powers of two: the scaled weights are exact
    got, sm2 = _layer(L, eps=0.0, w_dq=L.w_dq * 4.0, w_kv_a=wkv)
    assert rel_err(got, ref) < 1e-10 and np.allclose(sm2, sm, rtol=1e-10)
    wks = L.w_kv_a.copy()
    wks[R:] *= 8.0
    assert rel_err(_layer(L, eps=0.0, w_kv_a=wks)[0], ref) > 1e-3


def test_layer_zero_query_projection_gives_gated_prefix_mean():
    """W_UQ = 0 makes every visible score 0: token t of a sequence gets
    sigma(g_t) times the mean of V over the sequence's first t+1 tokens, and
    Delta_t is that times W_O^T."""
    L = _tiny_layer()
    d = L.dims
    H, R, N, V = d.heads, d.kv_rank, d.nope_dim, d.v_dim
    got, sm = _layer(L, w_uq=np.zeros_like(L.w_uq))
    ckv = oracle.rms_norm(oracle.linear(L.x, L.w_kv_a)[:, :R], L.g_kv, 1e-6)
    sig = 1.0 / (1.0 + np.exp(-oracle.linear(L.x, L.w_g)))
    want = np.zeros((L.ntok, H * V))
    for h in range(H):
        vh = ckv @ L.w_kv_b[h * (N + V) + N:(h + 1) * (N + V)].T
        for a, b in zip(L.cu_seqlens[:-1], L.cu_seqlens[1:]):
            csum = np.cumsum(vh[a:b], axis=0) / np.arange(1, b - a + 1)[:, None]
            want[a:b, h * V:(h + 1) * V] = csum
    want = (sig * want) @ L.w_o.T
    assert rel_err(got, want) < 1e-12
    assert np.all(sm == 0.0)


def test_layer_is_causal_within_each_sequence():
    """Changing token t of the second sequence changes Delta only at that
    sequence's rows from t on."""
    L = _tiny_layer()
    ref, _ = _layer(L)
    x2 = L.x.copy()
    t = 9 + 6
    x2[t] += 1.0
    got, _ = _layer(L, x=x2)
    diff = np.abs(got - ref).max(axis=1)
    assert np.all(diff[:t] == 0.0)
    assert np.all(diff[t:] > 0.0)


def test_layer_rows_equals_full_layer_on_listed_rows():
    L = synth.layer_inputs(synth.TINY, 40, 24, [9, 14], 7, bf16=True)
    args = (L.x, L.w_dq, L.g_q, L.w_uq, L.w_kv_a, L.g_kv, L.w_kv_b, L.w_g, L.w_o, L.cu_seqlens, L.dims, 1e-6)
    full, _ = oracle.layer_forward(*args)
    rows = [0, 8, 9, 15, 22]
    part = oracle.layer_rows(*args, rows)[0]
    assert np.array_equal(part, full[rows])


# ---------------------------------------------------------------------------
# QK-Clip
# ---------------------------------------------------------------------------


def _tiny_clip_case(T=24):
    dims = oracle.Dims(4, 16, 8, 16, 16)
    rng = np.random.default_rng(21)
    q_in = 20
    cq = rng.standard_normal((T, q_in))
    wq = rng.standard_normal((4 * 24, q_in)) / math.sqrt(q_in)
    ckv = rng.standard_normal((T, 16))
    ks = rng.standard_normal((T, 8))
    w = rng.standard_normal((4 * 32, 16)) / 4.0
    wq[1 * 24:2 * 24] *= 40.0
    w[1 * 32:1 * 32 + 16] *= 40.0
    return dims, cq, wq, ckv, ks, w


def test_qk_clip_scales_every_logit_of_a_clipped_head_by_gamma():
    dims, cq, wq, ckv, ks, w = _tiny_clip_case()
    T = cq.shape[0]
    q = oracle.q_projection(cq, wq, dims)
    _, probs0, sm = oracle.dense_prefill(q, ckv, ks, w, None, [0, T], dims)
    tau = 3.0 * np.sort(sm)[-2]     # only head 1 (x40) exceeds tau
    wq2, w2, mask, gamma = oracle.qk_clip(wq, w, sm, tau, dims)
    assert list(mask) == [False, True, False, False]
    assert gamma[1] == pytest.approx(tau / sm[1], rel=1e-15) and np.all(gamma[[0, 2, 3]] == 1.0)
    q2 = oracle.q_projection(cq, wq2, dims)
    # raw scaled logits before and after, for every head
    for h in range(4):
        kc, _ = oracle.expand_latent(ckv, w, dims, h)
        kc2, _ = oracle.expand_latent(ckv, w2, dims, h)
        S1 = q[:, h] @ np.concatenate([kc, ks], 1).T
        S2 = q2[:, h] @ np.concatenate([kc2, ks], 1).T
        assert np.allclose(S2, gamma[h] * S1, rtol=1e-12, atol=1e-12 * np.abs(S1).max())
    _, _, sm2 = oracle.prefill(q2, ckv, ks, w2, None, [0, T], dims)
    assert sm2[1] == pytest.approx(tau, rel=1e-12)
    # unclipped heads: same logits up to the BLAS's rounding order
    assert np.allclose(sm2[[0, 2, 3]], sm[[0, 2, 3]], rtol=1e-14, atol=0)
    # untouched: unclipped heads' rows, every V row
    for h in (0, 2, 3):
        assert np.array_equal(wq2[h * 24:(h + 1) * 24], wq[h * 24:(h + 1) * 24])
        assert np.array_equal(w2[h * 32:(h + 1) * 32], w[h * 32:(h + 1) * 32])
    assert np.array_equal(w2[32 + 16:64], w[32 + 16:64])


def test_qk_clip_threshold_is_strict():
    dims = oracle.Dims(5, 4, 2, 4, 4)
    rng = np.random.default_rng(3)
    wq = rng.standard_normal((5 * 6, 7))
    w = rng.standard_normal((5 * 8, 4))
    tau = 10.0
    sm = np.array([tau - 1e-9, tau, tau * (1 + 1e-12), -np.inf, 1e6])
    wq2, w2, mask, gamma = oracle.qk_clip(wq, w, sm, tau, dims)
    assert list(mask) == [False, False, True, False, True]
    assert gamma[4] == tau / 1e6 and gamma[3] == 1.0
    assert np.array_equal(wq2[:12], wq[:12])
    assert np.allclose(wq2[4 * 6:4 * 6 + 4], wq[4 * 6:4 * 6 + 4] * math.sqrt(1e-5), rtol=1e-15)
    assert np.allclose(wq2[4 * 6 + 4:5 * 6], wq[4 * 6 + 4:5 * 6] * 1e-5, rtol=1e-15)


def test_clip_stress_recipe_clips_exactly_the_scaled_heads():
    """The QK-Clip stress recipe at reduced length: the x40 heads reach logits
    above 1000 and are the only ones above tau = 100 (unscaled heads stay near 5)."""
    p = synth.clip_stress_inputs(synth.K3, 96, seed=3)
    q = synth.round_bf16(oracle.q_projection(p.cq, p.w_q_b, p.dims).astype(np.float32))
    sm = np.array([oracle.max_logit_head(q, p.ckv, p.ks, p.w_kv_b, p.cu_seqlens, p.dims, h)
                   for h in range(96)])
    mask = sm > synth.TAU
    assert list(np.nonzero(mask)[0]) == list(synth.CLIP_HEADS)
    assert sm[mask].min() > 1000.0
    assert sm[~mask].max() < 10.0


# ---------------------------------------------------------------------------
# QK-norm variant (per-head RMSNorm of the queries)
# ---------------------------------------------------------------------------


def test_qk_norm_query_closed_form_per_head():
    """q_h = [a 1_N, b 1_S] has root mean square sqrt((N a^2 + S b^2) / D):
    each head is divided by its own, then multiplied by the weight."""
    dims = synth.TINY
    H, N, S = dims.heads, dims.nope_dim, dims.shared_dim
    D = N + S
    ab = [(1.0, 2.0), (3.0, -0.5), (0.25, 0.0), (-7.0, 7.0)]
    q = np.zeros((2, H, D))
    for h, (a, b) in enumerate(ab):
        q[:, h, :N], q[:, h, N:] = a, b
    w = 1.0 + 0.1 * np.arange(D)
    for eps in (0.0, 0.5):
        got = oracle.qk_norm_query(q, w, eps, round_bf16=False)
        for h, (a, b) in enumerate(ab):
            r = math.sqrt((N * a * a + S * b * b) / D + eps)
            want = np.concatenate([np.full(N, a), np.full(S, b)]) / r * w
            assert np.allclose(got[0, h], want, rtol=1e-14, atol=0)
    assert np.array_equal(oracle.qk_norm_query(q, w, 0.0), oracle.round_to(oracle.qk_norm_query(q, w, 0.0, False),
                                                                             "bf16"))


def test_qk_norm_is_blind_to_the_query_scale():
    """Scaling any head's query by a positive factor leaves the output and the
    max logit unchanged (eps = 0; exactly so with bf16 rounding for powers of 2)."""
    dims = synth.TINY
    p = synth.prefill_inputs(dims, [19, 30], seed=31, bf16=True)
    w = 1.0 + 0.1 * np.random.default_rng(2).standard_normal(dims.nope_dim + dims.shared_dim)
    c = np.array([7.3, 0.01, 1.0, 250.0])[None, :, None]
    o1, l1, s1 = oracle.qk_norm_prefill(p.q, p.ckv, p.ks, p.w_kv_b, p.gate, p.cu_seqlens, dims, w, 0.0, False)
    o2, l2, s2 = oracle.qk_norm_prefill(p.q * c, p.ckv, p.ks, p.w_kv_b, p.gate, p.cu_seqlens, dims, w, 0.0, False)
    assert rel_err(o2, o1) < 1e-12 and np.allclose(s2, s1, rtol=1e-12)
    c2 = np.array([4.0, 0.125, 1.0, 1024.0])[None, :, None]
    o3, _, s3 = oracle.qk_norm_prefill(p.q * c2, p.ckv, p.ks, p.w_kv_b, p.gate, p.cu_seqlens, dims, w, 0.0)
    o4, _, s4 = oracle.qk_norm_prefill(p.q, p.ckv, p.ks, p.w_kv_b, p.gate, p.cu_seqlens, dims, w, 0.0)
    assert np.array_equal(o3, o4) and np.array_equal(s3, s4)
    # without the norm the same scaling changes everything
    o5, _, _ = oracle.prefill(p.q * c, p.ckv, p.ks, p.w_kv_b, p.gate, p.cu_seqlens, dims)
    assert rel_err(o5, oracle.prefill(p.q, p.ckv, p.ks, p.w_kv_b, p.gate, p.cu_seqlens, dims)[0]) > 1e-2


def test_qk_norm_of_unit_rms_queries_is_the_plain_prefill():
    dims = synth.TINY
    p = synth.prefill_inputs(dims, [25], seed=32, bf16=False)
    q = np.asarray(p.q, dtype=np.float64)
    q = q / np.sqrt(np.mean(q * q, axis=-1, keepdims=True))
    ref = oracle.prefill(q, p.ckv, p.ks, p.w_kv_b, p.gate, p.cu_seqlens, dims)
    got = oracle.qk_norm_prefill(q, p.ckv, p.ks, p.w_kv_b, p.gate, p.cu_seqlens, dims, None, 0.0, False)
    assert rel_err(got[0], ref[0]) < 1e-12 and np.allclose(got[2], ref[2], rtol=1e-12)
    # decode with the norm equals the last rows of prefill with the norm
    rows = [np.concatenate([p.ckv, p.ks], axis=1)]
    out, sm = oracle.qk_norm_absorbed(p.q[None, -2:], rows, p.w_kv_b, p.gate[None, -2:], dims, None, 1e-6, False)
    full = oracle.qk_norm_prefill(p.q, p.ckv, p.ks, p.w_kv_b, p.gate, p.cu_seqlens, dims, None, 1e-6, False)[0]
    assert rel_err(out[0], full[-2:]) < 1e-10


def test_qk_norm_logit_bound_holds_and_is_attained():
    """Every logit stays within the closed-form bound; a constructed input
    (latent along W_UK_h's top right singular vector, query along the key it
    makes) reaches it exactly."""
    dims = synth.TINY
    H, R, S, N, V = dims.heads, dims.kv_rank, dims.shared_dim, dims.nope_dim, dims.v_dim
    D = N + S
    rng = np.random.default_rng(33)
    p = synth.prefill_inputs(dims, [40], seed=33, bf16=False)
    ckv = p.ckv / np.sqrt(np.mean(p.ckv.astype(np.float64) ** 2, axis=1, keepdims=True))   # unit-RMS entries
    ks = p.ks / np.sqrt(np.mean(p.ks.astype(np.float64) ** 2, axis=1, keepdims=True))
    w = 1.0 + 0.2 * rng.standard_normal(D)
    bound = oracle.qk_norm_logit_bound(p.w_kv_b, dims, w, math.sqrt(R), math.sqrt(S))
    qn = oracle.qk_norm_query(p.q, w, 0.0, False)
    _, probs, sm = oracle.dense_prefill(qn, ckv, ks, p.w_kv_b, None, p.cu_seqlens, dims)
    assert np.all(sm <= bound) and np.all(sm > 0.05 * bound)
    # attainment: one token whose latent is sqrt(R) times the top right singular vector of W_UK_h
    h = 2
    wk = np.asarray(p.w_kv_b, dtype=np.float64)[h * (N + V):h * (N + V) + N]      # [N, R]
    _, sv, vt = np.linalg.svd(wk)
    c = math.sqrt(R) * vt[0]
    k = np.ones(S)                                                               # unit RMS
    key = np.concatenate([c @ wk.T, k])
    q = np.ones((1, H, D))
    q[0, h] = key
    one = np.array([0, 1], dtype=np.int32)
    sm1 = oracle.max_logit_head(oracle.qk_norm_query(q, None, 0.0, False), c[None], k[None], p.w_kv_b, one, dims, h)
    b1 = oracle.qk_norm_logit_bound(p.w_kv_b, dims, None, math.sqrt(R), math.sqrt(S))[h]
    assert sm1 == pytest.approx(b1, rel=1e-12)
    assert b1 == pytest.approx(math.sqrt(sv[0] ** 2 * R + S), rel=1e-12)


def test_qk_norm_ignores_a_scaled_query_weight_but_not_a_scaled_key_weight():
    """The clip-stress mechanism under the norm: scaling a head's q_b_proj
    rows x40 changes none of its logits, while scaling its W_UK rows x40 (with
    k^S = 0, so every logit comes through W_UK) multiplies every logit of the
    head by exactly 40. The norm on the inputs does not bound the logit
    through the key up-projection."""
    dims = synth.Dims(4, 32, 16, 32, 32)
    H, N, V, S, D = 4, 32, 32, 16, 48
    p = synth.clip_stress_inputs(dims, 24, seed=34, q_in=64, heads=(1,), factor=1.0)
    ks0 = np.zeros_like(p.ks)
    q = oracle.q_projection(p.cq, p.w_q_b, dims)
    wq40 = np.array(p.w_q_b, dtype=np.float64)
    wq40[1 * D:2 * D] *= 40.0
    q40 = oracle.q_projection(p.cq, wq40, dims)
    wk40 = np.array(p.w_kv_b, dtype=np.float64)
    wk40[1 * (N + V):1 * (N + V) + N] *= 40.0

    def smax(qq, wk, ks):
        return oracle.qk_norm_prefill(qq, p.ckv, ks, wk, None, p.cu_seqlens, dims, None, 0.0, False)[2]
    base = smax(q, p.w_kv_b, ks0)
    assert np.allclose(smax(q40, p.w_kv_b, ks0), base, rtol=1e-12)
    s40 = smax(q, wk40, ks0)
    assert s40[1] == pytest.approx(40.0 * base[1], rel=1e-12)
    assert np.array_equal(np.delete(s40, 1), np.delete(base, 1))
    # without the norm the query weight's x40 multiplies the logits as well
    plain = oracle.prefill(q40, p.ckv, ks0, p.w_kv_b, None, p.cu_seqlens, dims)[2]
    assert plain[1] == pytest.approx(40.0 * oracle.prefill(q, p.ckv, ks0, p.w_kv_b, None, p.cu_seqlens, dims)[2][1],
                                     rel=1e-12)
