"""Plain float64 CPU oracle for gated, no-position MLA (test infrastructure only).

Sources (cited by page title and section):
  [MLA]  "Kimi K3 · Gated MLA · OpenModelAtlas": the 20-step equation list
         (query heads, key and value heads, causal attention, gate), the
         ``KimiMLAAttention`` constructor/forward excerpts and the
         ``eager_attention_forward`` excerpt (fp32 softmax, scaling = q_head_dim^-1/2).
  [FR]   "Gated MLA et NoPE" (mkdocs.reaper.mx): cache row of 512 + 64 values,
         sigmoid output gate, no position encoding.
  [CLIP] "SOTA-131" practice page (anthology-of-the-sota): QK-Clip rescales a
         head's query and key projection weights when its maximum logit exceeds
         a threshold.
  [FW]   "Kimi Qkclip" (Fireworks blog): training materialises K, inference
         skips the K up-projection (the absorbed form).

Conventions shared with the library's C ABI (layouts, not arithmetic):
  q [Ntok, H, D] with D = N + S (first N = q^C, last S = q^R), c^KV [Ntok, R],
  k^S [Ntok, S], kv_b_proj.weight [H*(N+V), R] (head h: N rows of W_UK_h^T then
  V rows of W_UV_h^T), gate logits [Ntok, H*V], output [Ntok, H*V] head-major.

Everything is computed in float64 from the exact values of the inputs. No
function here is blocked, fused or reordered beyond splitting independent
query rows into blocks to bound memory; each query row is computed from its
full masked score row exactly as the equations define it.
"""
from __future__ import annotations

import collections
import math

import numpy as np

Dims = collections.namedtuple("Dims", "heads kv_rank shared_dim nope_dim v_dim")

f64 = np.float64


def _dims(d) -> Dims:
    return Dims(int(d.heads), int(d.kv_rank), int(d.shared_dim), int(d.nope_dim), int(d.v_dim))


def scale_of(d) -> float:
    """The score scale 1/sqrt(q_head_dim), q_head_dim = nope + shared ([MLA]
    constructor: ``self.scaling = self.q_head_dim ** (-0.5)``; equation S <- S/sqrt(192))."""
    d = _dims(d)
    return 1.0 / math.sqrt(d.nope_dim + d.shared_dim)


def sigmoid(x):
    """sigma(x) = 1 / (1 + e^{-x})  ([MLA] gate step o = sigma(g) . o~)."""
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-np.asarray(x, dtype=f64)))


# ---------------------------------------------------------------------------
# Key and value heads ([MLA] steps "[k^C v] = c^KV W_UKV", K^C_h = cols 1:128,
# V_h = cols 129:256, K_h = [K^C_h k^S])
# ---------------------------------------------------------------------------


def expand_latent(ckv, w_kv_b, dims, head: int):
    """K^C_h and V_h of one head from the latent c^KV.

    [k^C v] = c^KV W_UKV with W_UKV = kv_b_proj.weight^T; head h's block of 256
    output columns splits into its first N (K^C_h) and its last V (V_h).
    Returns (K^C_h [T, N], V_h [T, V]) in float64.
    """
    d = _dims(dims)
    w = np.asarray(w_kv_b, dtype=f64)
    blk = w[head * (d.nope_dim + d.v_dim):(head + 1) * (d.nope_dim + d.v_dim), :]   # [N+V, R]
    kv = np.asarray(ckv, dtype=f64) @ blk.T                                          # [T, N+V]
    return kv[:, :d.nope_dim], kv[:, d.nope_dim:]


def key_of_head(kc_h, ks):
    """K_h = [K^C_h, k^S]: the shared k^S is the same for every head."""
    return np.concatenate([np.asarray(kc_h, dtype=f64), np.asarray(ks, dtype=f64)], axis=1)


# ---------------------------------------------------------------------------
# Causal attention ([MLA] steps S = Q K^T, S <- S/sqrt(192), causal softmax,
# O~ = A V, reshape, gate)
# ---------------------------------------------------------------------------


def _attend_sequence(Q, K, Vv, scale, block):
    """One sequence and one head: rows of A over s <= t, then A V.

    Returns (O~ [L, V], lse [L], max unmasked scaled logit).
    """
    L = Q.shape[0]
    out = np.zeros((L, Vv.shape[1]), dtype=f64)
    lse = np.full(L, -np.inf, dtype=f64)
    smax = -np.inf
    for t0 in range(0, L, block):
        t1 = min(L, t0 + block)
        S = (Q[t0:t1] @ K[:t1].T) * scale               # S = Q K^T / sqrt(D)
        t = np.arange(t0, t1)[:, None]
        s = np.arange(t1)[None, :]
        visible = s <= t                                # causal: s <= t
        S = np.where(visible, S, -np.inf)
        smax = max(smax, float(S.max()))
        m = S.max(axis=1, keepdims=True)
        e = np.exp(S - m)                               # exp S_{t,s}; exactly 0 where s > t
        den = e.sum(axis=1, keepdims=True)              # sum_{u <= t} exp S_{t,u}
        A = e / den
        out[t0:t1] = A @ Vv[:t1]                        # O~ = A V
        lse[t0:t1] = (m + np.log(den))[:, 0]
    return out, lse, smax


def prefill(q, ckv, ks, w_kv_b, gate, cu_seqlens, dims, block: int = 512, heads=None):
    """Training-form gated MLA over packed sequences.

    For every head h and every sequence [a, b) of ``cu_seqlens``:
    K^C_h, V_h from c^KV (expansion), K_h = [K^C_h, k^S], S = Q_h K_h^T / sqrt(D),
    causal softmax (A = 0 for s > t), O~ = A V_h. Sequences never attend to
    each other. Then o~ = reshape(O~) head-major and o = sigma(g) . o~ (no gate
    when ``gate`` is None).

    Returns (out [Ntok, H*V], lse [H, Ntok] natural log, max_logit [H]) in
    float64; max_logit[h] is the largest scaled logit S_{t,s} over every
    unmasked pair of every sequence (-inf when there is none).
    """
    d = _dims(dims)
    H, N, V = d.heads, d.nope_dim, d.v_dim
    cu = [int(x) for x in cu_seqlens]
    n = cu[-1]
    scale = scale_of(d)
    q = np.asarray(q)
    out = np.zeros((n, H * V), dtype=f64)
    lse = np.full((H, n), -np.inf, dtype=f64)
    smax = np.full(H, -np.inf, dtype=f64)
    for h in (range(H) if heads is None else heads):
        kc, vv = expand_latent(ckv, w_kv_b, d, h)
        K = key_of_head(kc, ks)
        Q = np.asarray(q[:, h, :], dtype=f64)
        for a, b in zip(cu[:-1], cu[1:]):
            if b <= a:
                continue
            o, l, m = _attend_sequence(Q[a:b], K[a:b], vv[a:b], scale, block)
            out[a:b, h * V:(h + 1) * V] = o
            lse[h, a:b] = l
            smax[h] = max(smax[h], m)
    if gate is not None:
        out = sigmoid(gate) * out
    return out, lse, smax


def max_logit_head(q, ckv, ks, w_kv_b, cu_seqlens, dims, head: int, block: int = 1024):
    """Largest scaled causal logit of one head over all sequences (no softmax)."""
    d = _dims(dims)
    scale = scale_of(d)
    kc, _ = expand_latent(ckv, w_kv_b, d, head)
    K = key_of_head(kc, ks)
    Q = np.asarray(np.asarray(q)[:, head, :], dtype=f64)
    cu = [int(x) for x in cu_seqlens]
    best = -np.inf
    for a, b in zip(cu[:-1], cu[1:]):
        for t0 in range(a, b, block):
            t1 = min(b, t0 + block)
            S = (Q[t0:t1] @ K[a:t1].T) * scale
            t = np.arange(t0, t1)[:, None]
            s = np.arange(a, t1)[None, :]
            S = np.where(s <= t, S, -np.inf)
            best = max(best, float(S.max()))
    return best


def prefill_rows(q, ckv, ks, w_kv_b, gate, cu_seqlens, dims, head: int, rows):
    """Selected output rows of one head (for spot checks at sizes the full
    oracle cannot finish). ``rows`` are global token indices.

    Returns (o [len(rows), V] gated, lse [len(rows)]).
    """
    d = _dims(dims)
    V = d.v_dim
    scale = scale_of(d)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    kc, vv = expand_latent(ckv, w_kv_b, d, head)
    K = key_of_head(kc, ks)
    qq = np.asarray(q)
    out = np.zeros((len(rows), V), dtype=f64)
    lse = np.zeros(len(rows), dtype=f64)
    for i, t in enumerate(rows):
        s_idx = int(np.searchsorted(cu, t, side="right") - 1)
        a = int(cu[s_idx])
        S = (K[a:t + 1] @ np.asarray(qq[t, head, :], dtype=f64)) * scale   # s = a..t
        m = S.max()
        e = np.exp(S - m)
        den = e.sum()
        o = (e / den) @ vv[a:t + 1]
        if gate is not None:
            o = sigmoid(np.asarray(gate)[t, head * V:(head + 1) * V]) * o
        out[i] = o
        lse[i] = m + math.log(den)
    return out, lse


def dense_prefill(q, ckv, ks, w_kv_b, gate, cu_seqlens, dims):
    """Brute force for tiny inputs, in the style of ``eager_attention_forward``.

    Materialises every head's full K and V with one einsum, builds the whole
    Ntok x Ntok score matrix per head, adds an additive mask (0 where the key is
    in the same sequence and not after the query, -inf elsewhere), and applies
    a textbook softmax. Returns (out [Ntok, H*V], probs [H, Ntok, Ntok],
    max_logit [H]).
    """
    d = _dims(dims)
    H, N, V, S_ = d.heads, d.nope_dim, d.v_dim, d.shared_dim
    n = int(cu_seqlens[-1])
    w = np.asarray(w_kv_b, dtype=f64).reshape(H, N + V, -1)                 # [H, N+V, R]
    kv = np.einsum("tr,hcr->htc", np.asarray(ckv, dtype=f64), w)           # [H, T, N+V]
    kc, vv = kv[..., :N], kv[..., N:]
    ksb = np.broadcast_to(np.asarray(ks, dtype=f64)[None], (H, n, S_))
    key = np.concatenate([kc, ksb], axis=-1)                               # [H, T, D]
    qh = np.asarray(q, dtype=f64).transpose(1, 0, 2)                       # [H, T, D]
    seq_id = np.repeat(np.arange(len(cu_seqlens) - 1), np.diff(np.asarray(cu_seqlens)))
    pos = np.arange(n)
    allowed = (seq_id[:, None] == seq_id[None, :]) & (pos[None, :] <= pos[:, None])
    mask = np.where(allowed, 0.0, -np.inf)
    scores = np.einsum("hqd,hkd->hqk", qh, key) * scale_of(d) + mask[None]
    smax = np.where(allowed[None], scores, -np.inf).reshape(H, -1).max(axis=1)
    ex = np.exp(scores - scores.max(axis=-1, keepdims=True))
    probs = ex / ex.sum(axis=-1, keepdims=True)
    o = np.einsum("hqk,hkd->qhd", probs, vv).reshape(n, H * V)
    if gate is not None:
        o = o / (1.0 + np.exp(-np.asarray(gate, dtype=f64)))
    return o, probs, smax


# ---------------------------------------------------------------------------
# Absorbed (inference) form ([FW] "the projection is skipped" at decode; the
# cache row [c^KV | k^S] of [FR]). By associativity of the [MLA] equations:
#   q^C . K^C_s = c_s . (W_UK_h q^C)   and   sum_s p_s V_s = (sum_s p_s c_s) W_UV_h
# ---------------------------------------------------------------------------


def absorb_query(q_h, w_kv_b, dims, head: int):
    """q_abs = [W_UK_h q^C_h, q^R_h] (length R + S) for one head and one token."""
    d = _dims(dims)
    N, V = d.nope_dim, d.v_dim
    w = np.asarray(w_kv_b, dtype=f64)
    wk = w[head * (N + V):head * (N + V) + N, :]             # [N, R] = W_UK_h^T
    q_h = np.asarray(q_h, dtype=f64)
    return np.concatenate([wk.T @ q_h[:N], q_h[N:]])


def absorbed(q, cache_rows, w_kv_b, gate, dims):
    """Absorbed-form gated MLA over a latent cache.

    q [B, Tq, H, D]; ``cache_rows[b]`` holds the valid rows [c^KV | k^S] of
    sequence b ([L_b, R+S]); gate [B, Tq, H*V] or None. Query i of Tq sees rows
    j <= L_b - Tq + i (the Tq queries are the last Tq positions of the
    sequence). Scores use the same 1/sqrt(N+S) scale as the training form.

    Returns (out [B, Tq, H*V], max_logit [H]).
    """
    d = _dims(dims)
    H, R, N, V = d.heads, d.kv_rank, d.nope_dim, d.v_dim
    scale = scale_of(d)
    q = np.asarray(q)
    B, Tq = q.shape[0], q.shape[1]
    w = np.asarray(w_kv_b, dtype=f64)
    out = np.zeros((B, Tq, H * V), dtype=f64)
    smax = np.full(H, -np.inf, dtype=f64)
    for b in range(B):
        rows = np.asarray(cache_rows[b], dtype=f64)          # [L, R+S]
        L = rows.shape[0]
        for i in range(Tq):
            vis = L - Tq + i + 1
            if vis <= 0:
                continue
            for h in range(H):
                qa = absorb_query(q[b, i, h], w, d, h)
                s = (rows[:vis] @ qa) * scale
                smax[h] = max(smax[h], float(s.max()))
                m = s.max()
                e = np.exp(s - m)
                p = e / e.sum()
                o_lat = p @ rows[:vis, :R]                   # sum_s p_s c_s
                wv = w[h * (N + V) + N:(h + 1) * (N + V), :]  # [V, R] = W_UV_h^T
                out[b, i, h * V:(h + 1) * V] = wv @ o_lat    # (o_lat) W_UV_h
    if gate is not None:
        out = sigmoid(gate) * out
    return out, smax


def absorbed_max_logit(q, cache_rows, w_kv_b, dims):
    """Per-head maximum scaled logit of the absorbed form, without the softmax.

    The same logits as ``absorbed``: s_j = scale * q_abs . [c^KV_j | k^S_j] with
    q_abs = [W_UK_h q^C, q^R] (associativity of the [MLA] score step with the
    key expansion), over the visible rows j <= L_b - Tq + i of every query i of
    every sequence b. Sequences are taken one at a time, so a workload whose
    cache is too large to hold whole can pass ``cache_rows`` as any indexable
    whose item b returns sequence b's rows. Returns max_logit [H] (float64).
    """
    d = _dims(dims)
    H = d.heads
    scale = scale_of(d)
    q = np.asarray(q)
    B, Tq = q.shape[0], q.shape[1]
    w = np.asarray(w_kv_b, dtype=f64)
    smax = np.full(H, -np.inf, dtype=f64)
    for b in range(B):
        rows = np.asarray(cache_rows[b], dtype=f64)
        L = rows.shape[0]
        for i in range(Tq):
            vis = L - Tq + i + 1
            if vis <= 0:
                continue
            qa = np.stack([absorb_query(q[b, i, h], w, d, h) for h in range(H)])   # [H, R+S]
            s = (rows[:vis] @ qa.T) * scale                                         # [vis, H]
            smax = np.maximum(smax, s.max(axis=0))
    return smax


def absorbed_rows_selected(q, cache_rows, w_kv_b, gate, dims, batches):
    """``absorbed`` restricted to the listed sequences (spot checks)."""
    qs = np.asarray(q)[list(batches)]
    gs = None if gate is None else np.asarray(gate)[list(batches)]
    return absorbed(qs, [cache_rows[b] for b in batches], w_kv_b, gs, dims)


# ---------------------------------------------------------------------------
# Expanded-cache decode: the materialised K_h = [K^C_h, k^S] and V_h of every
# cached token kept per head, as the training form builds them ([MLA] steps
# "[k^C v] = c^KV W_UKV" and "K_h = [K^C_h k^S]"), instead of the single latent
# row of [FR]. Attention over it is the [MLA] equation list for the last Tq
# query positions.
# ---------------------------------------------------------------------------


def expanded_cache(cache_rows, w_kv_b, dims):
    """Per-head K and V of every cached token from latent rows [c^KV | k^S].

    ``cache_rows[b]`` is [L_b, R+S]. Returns lists ``k_rows[b]`` [H, L_b, N+S]
    and ``v_rows[b]`` [H, L_b, V] in float64.
    """
    d = _dims(dims)
    R = d.kv_rank
    k_rows, v_rows = [], []
    for rows in cache_rows:
        rows = np.asarray(rows, dtype=f64)
        ks, vs = [], []
        for h in range(d.heads):
            kc, vv = expand_latent(rows[:, :R], w_kv_b, d, h)
            ks.append(key_of_head(kc, rows[:, R:]))
            vs.append(vv)
        k_rows.append(np.stack(ks))
        v_rows.append(np.stack(vs))
    return k_rows, v_rows


def expanded(q, k_rows, v_rows, gate, dims):
    """Gated MLA decode over a per-head (expanded) cache.

    q [B, Tq, H, D]; ``k_rows[b]`` [H, L_b, D] and ``v_rows[b]`` [H, L_b, V]
    hold the valid rows of sequence b; gate [B, Tq, H*V] or None. Query i of Tq
    sees rows j <= L_b - Tq + i, with the scale 1/sqrt(N+S):
      s_j = scale * q[b, i, h] . K_h[j],  p = softmax(s),  O~_h = sum_j p_j V_h[j],
      out = sigma(g) . O~.
    Returns (out [B, Tq, H*V], max_logit [H]).
    """
    d = _dims(dims)
    H, V = d.heads, d.v_dim
    scale = scale_of(d)
    q = np.asarray(q)
    B, Tq = q.shape[0], q.shape[1]
    out = np.zeros((B, Tq, H * V), dtype=f64)
    smax = np.full(H, -np.inf, dtype=f64)
    for b in range(B):
        K = np.asarray(k_rows[b], dtype=f64)
        Vv = np.asarray(v_rows[b], dtype=f64)
        L = K.shape[1]
        for i in range(Tq):
            vis = L - Tq + i + 1
            if vis <= 0:
                continue
            for h in range(H):
                s = (K[h, :vis] @ np.asarray(q[b, i, h], dtype=f64)) * scale
                smax[h] = max(smax[h], float(s.max()))
                e = np.exp(s - s.max())
                p = e / e.sum()
                out[b, i, h * V:(h + 1) * V] = p @ Vv[h, :vis]
    if gate is not None:
        out = sigmoid(gate) * out
    return out, smax


# ---------------------------------------------------------------------------
# Backward of the training-form prefill: the gradients of the [MLA] equation
# list (expansion, key assembly, scaled causal softmax, value mix, gate) with
# respect to q, c^KV, k^S, kv_b_proj.weight and the gate logits, for an
# upstream gradient dO of the output o. Chain rule through
#   o = sigma(g) . O~,  O~ = A V,  A = softmax(S) (causal),  S = scale Q K^T,
#   K = [K^C, k^S],  [K^C V] = c^KV W_UKV.
# ---------------------------------------------------------------------------


def prefill_backward(q, ckv, ks, w_kv_b, gate, cu_seqlens, dims, dout):
    """Returns (dq [Ntok, H, D], dckv [Ntok, R], dks [Ntok, S], dw_kv_b
    [H*(N+V), R], dgate [Ntok, H*V] or None), all float64.

    Per head and sequence, with P the causal softmax rows:
      dO~ = dO . sigma(g),  dg = dO . O~ . sigma(g) (1 - sigma(g)),
      dV = P^T dO~,  dP = dO~ V^T,  dS = P . (dP - rowsum(dP . P)),
      dQ = scale dS K,  dK = scale dS^T Q;
    then dK^C, dV flow back through W_UKV into c^KV and the weight, and the
    k^S part of dK sums over the heads.
    """
    d = _dims(dims)
    H, R, S_, N, V = d.heads, d.kv_rank, d.shared_dim, d.nope_dim, d.v_dim
    scale = scale_of(d)
    cu = [int(x) for x in cu_seqlens]
    n = cu[-1]
    q = np.asarray(q, dtype=f64)
    c = np.asarray(ckv, dtype=f64)
    w = np.asarray(w_kv_b, dtype=f64)
    dout = np.asarray(dout, dtype=f64)
    sig = sigmoid(gate) if gate is not None else np.ones((n, H * V))
    dq = np.zeros((n, H, N + S_))
    dckv = np.zeros((n, R))
    dks = np.zeros((n, S_))
    dw = np.zeros_like(w)
    dgate = np.zeros((n, H * V)) if gate is not None else None
    for h in range(H):
        kc, vv = expand_latent(c, w, d, h)
        K = key_of_head(kc, ks)
        cols = slice(h * V, (h + 1) * V)
        dKh = np.zeros((n, N + S_))
        dVh = np.zeros((n, V))
        for a, b in zip(cu[:-1], cu[1:]):
            if b <= a:
                continue
            Q = q[a:b, h]
            Sm = (Q @ K[a:b].T) * scale
            Sm = np.where(np.tril(np.ones((b - a, b - a), dtype=bool)), Sm, -np.inf)
            P = np.exp(Sm - Sm.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            Ot = P @ vv[a:b]                                    # O~ of this head
            dOt = dout[a:b, cols] * sig[a:b, cols]
            if dgate is not None:
                dgate[a:b, cols] = dout[a:b, cols] * Ot * sig[a:b, cols] * (1.0 - sig[a:b, cols])
            dVh[a:b] = P.T @ dOt
            dP = dOt @ vv[a:b].T
            dS = P * (dP - np.sum(dP * P, axis=1, keepdims=True))
            dq[a:b, h] = scale * (dS @ K[a:b])
            dKh[a:b] = scale * (dS.T @ Q)
        blk = slice(h * (N + V), (h + 1) * (N + V))
        dkv = np.concatenate([dKh[:, :N], dVh], axis=1)           # d[K^C_h V_h]
        dckv += dkv @ w[blk]
        dw[blk] += dkv.T @ c
        dks += dKh[:, N:]
    return dq, dckv, dks, dw, dgate


# ---------------------------------------------------------------------------
# The whole gated MLA layer ([MLA] equation list, all 20 steps, and the
# KimiMLAAttention constructor/forward excerpts): q_a_proj -> q_a_layernorm ->
# q_b_proj; kv_a_proj_with_mqa -> [c^KV | k^S] -> kv_a_layernorm on c^KV;
# g_proj; attention; o_proj. Every projection is nn.Linear without bias.
# ---------------------------------------------------------------------------


def linear(x, weight):
    """nn.Linear without bias: y = x W^T, W = weight [out, in]."""
    return np.asarray(x, dtype=f64) @ np.asarray(weight, dtype=f64).T


def rms_norm(x, weight, eps: float):
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps), times the
    learned per-feature weight. (The pages name KimiRMSNorm without printing
    it; this is the standard definition, with eps a parameter.)"""
    x = np.asarray(x, dtype=f64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x * r * np.asarray(weight, dtype=f64)


def layer_forward(x, w_dq, g_q, w_uq, w_kv_a, g_kv, w_kv_b, w_g, w_o, cu_seqlens, dims, eps: float,
                  round_bf16: bool = True):
    """Delta_attn for packed sequences: the [MLA] equation list end to end.

      c^Q = x W_DQ,  c^Q^ = RMSNorm(c^Q),  q = c^Q^ W_UQ  (q_b_proj),
      [c^KV | k^S] = x W_DKV,  c^KV^ = RMSNorm(c^KV),
      g = x W_g,  o = sigma(g) . attention(q, c^KV^, k^S)  (``prefill``),
      Delta = o W_O.

    x [Ntok, hidden]; weights in the nn.Linear layout [out, in]: w_dq
    [q_rank, hidden], w_uq [H*D, q_rank], w_kv_a [R+S, hidden], w_kv_b
    [H*(N+V), R], w_g [H*V, hidden], w_o [hidden, H*V]; g_q [q_rank] and g_kv
    [R] are the RMSNorm weights. With ``round_bf16`` every activation that the
    model keeps in its bf16 dtype (each projection's output and each norm's
    output) is rounded to bf16 (nearest-even) where it is produced; the
    arithmetic itself stays float64.

    Returns (Delta [Ntok, hidden], max_logit [H]).
    """
    d = _dims(dims)
    H, R, D = d.heads, d.kv_rank, d.nope_dim + d.shared_dim
    rnd = (lambda a: round_to(a, "bf16")) if round_bf16 else (lambda a: np.asarray(a, dtype=f64))
    n = np.asarray(x).shape[0]
    cq = rnd(linear(x, w_dq))
    q = rnd(linear(rnd(rms_norm(cq, g_q, eps)), w_uq)).reshape(n, H, D)
    ckv_ks = rnd(linear(x, w_kv_a))
    ckv = rnd(rms_norm(ckv_ks[:, :R], g_kv, eps))
    ks = ckv_ks[:, R:]
    g = rnd(linear(x, w_g))
    o, _, smax = prefill(q, ckv, ks, w_kv_b, g, cu_seqlens, d)
    return linear(rnd(o), w_o), smax


def layer_rows(x, w_dq, g_q, w_uq, w_kv_a, g_kv, w_kv_b, w_g, w_o, cu_seqlens, dims, eps: float, rows,
               round_bf16: bool = True):
    """``layer_forward`` for the listed global token rows only (spot checks at
    sizes the full oracle cannot finish): q, c^KV^ and k^S are formed for every
    token (the rows attend to their whole prefix), the gate and the output only
    for the listed rows.

    Returns (Delta [len(rows), hidden], q [Ntok, H, D], c^KV^ [Ntok, R], k^S [Ntok, S]).
    """
    d = _dims(dims)
    H, R, V, D = d.heads, d.kv_rank, d.v_dim, d.nope_dim + d.shared_dim
    rnd = (lambda a: round_to(a, "bf16")) if round_bf16 else (lambda a: np.asarray(a, dtype=f64))
    n = np.asarray(x).shape[0]
    rows = [int(t) for t in rows]
    q = rnd(linear(rnd(rms_norm(rnd(linear(x, w_dq)), g_q, eps)), w_uq)).reshape(n, H, D)
    ckv_ks = rnd(linear(x, w_kv_a))
    ckv = rnd(rms_norm(ckv_ks[:, :R], g_kv, eps))
    ks = ckv_ks[:, R:]
    g = np.zeros((n, H * V), dtype=f64)
    g[rows] = rnd(linear(np.asarray(x)[rows], w_g))
    o = np.zeros((len(rows), H * V), dtype=f64)
    for h in range(H):
        o[:, h * V:(h + 1) * V] = prefill_rows(q, ckv, ks, w_kv_b, g, cu_seqlens, d, h, rows)[0]
    return linear(rnd(o), w_o), q, ckv, ks


# ---------------------------------------------------------------------------
# QK-norm variant ([CLIP] "Variations": the other route to bounded logits,
# an RMSNorm on the attention queries and on the KV entries instead of a clip
# of the weights; "Mechanism": the norm bounds the input of the logit). In
# this MLA the compressed entry c^KV already leaves an RMSNorm
# (kv_a_layernorm) and k^S is normalised where it is produced, so the
# attention calls take them as given; the query is normalised per head.
# ---------------------------------------------------------------------------


def qk_norm_query(q, weight, eps: float, round_bf16: bool = True):
    """Per-head RMSNorm of the queries: each head's D = N + S query features
    (q^C and q^R together) divided by their root mean square, times the
    per-feature weight [D] shared by the heads (None = ones). With
    ``round_bf16`` the normalised query is rounded to bf16 where it is
    produced, as every activation the model keeps in its dtype.

    q [..., H, D] -> same shape, float64.
    """
    q = np.asarray(q, dtype=f64)
    w = np.ones(q.shape[-1]) if weight is None else np.asarray(weight, dtype=f64)
    y = rms_norm(q, w, eps)
    return round_to(y, "bf16") if round_bf16 else y


def qk_norm_prefill(q, ckv, ks, w_kv_b, gate, cu_seqlens, dims, q_norm_weight, eps: float,
                    round_bf16: bool = True, heads=None):
    """The training-form prefill on per-head normalised queries: first
    ``qk_norm_query``, then ``prefill`` unchanged (c^KV and k^S as given)."""
    qn = qk_norm_query(q, q_norm_weight, eps, round_bf16)
    return prefill(qn, ckv, ks, w_kv_b, gate, cu_seqlens, dims, heads=heads)


def qk_norm_absorbed(q, cache_rows, w_kv_b, gate, dims, q_norm_weight, eps: float, round_bf16: bool = True):
    """The absorbed form on per-head normalised queries (``qk_norm_query``,
    then ``absorbed``)."""
    qn = qk_norm_query(q, q_norm_weight, eps, round_bf16)
    return absorbed(qn, cache_rows, w_kv_b, gate, dims)


def qk_norm_logit_bound(w_kv_b, dims, q_norm_weight, ckv_norm_max: float, ks_norm_max: float):
    """Closed-form bound of every scaled logit of each head under the QK-norm
    variant (with eps = 0):

      |S| = |q_n^C . (c W_UK_h) + q_n^R . k^S| / sqrt(D)
          <= ||q_n|| sqrt(||c W_UK_h||^2 + ||k^S||^2) / sqrt(D)          (Cauchy-Schwarz)
          <= max|w| sqrt(sigma_h^2 ||c||^2 + ||k^S||^2),

    since ||q_n|| <= sqrt(D) max|w|, with sigma_h the largest singular value
    of W_UK_h and ||c||, ||k^S|| the largest entry norms. It grows with
    sigma_h: the norm of the inputs does not bound the logit through the
    key up-projection. Returns [H] (float64).
    """
    d = _dims(dims)
    H, N, V = d.heads, d.nope_dim, d.v_dim
    w = np.asarray(w_kv_b, dtype=f64)
    wmax = 1.0 if q_norm_weight is None else float(np.max(np.abs(np.asarray(q_norm_weight, dtype=f64))))
    out = np.zeros(H)
    for h in range(H):
        sigma = np.linalg.norm(w[h * (N + V):h * (N + V) + N, :], 2)   # largest singular value of W_UK_h
        out[h] = wmax * math.sqrt(sigma ** 2 * ckv_norm_max ** 2 + ks_norm_max ** 2)
    return out


# ---------------------------------------------------------------------------
# Query projection ([MLA] "q = c^Q W_UQ") and QK-Clip ([CLIP])
# ---------------------------------------------------------------------------


def q_projection(cq, w_q_b, dims):
    """q = c^Q W_UQ with W_UQ = q_b_proj.weight^T, viewed [Ntok, H, D]."""
    d = _dims(dims)
    q = np.asarray(cq, dtype=f64) @ np.asarray(w_q_b, dtype=f64).T
    return q.reshape(q.shape[0], d.heads, d.nope_dim + d.shared_dim)


def qk_clip(w_q_b, w_kv_b, max_logit, tau, dims):
    """QK-Clip: for each head whose maximum logit exceeds tau, rescale that
    head's query and key projection weights so the maximum becomes tau.

    gamma_h = tau / S_max[h] when S_max[h] > tau, else 1. Every logit of head h
    is q^C.K^C + q^R.k^S (then scaled); k^S is shared by all heads and is left
    untouched, so the head's q^R rows take the whole factor gamma_h, and the
    head-specific nope parts take sqrt(gamma_h) on each side (q^C rows of
    q_b_proj and K^C rows of kv_b_proj). Then every logit of head h is exactly
    gamma_h times its old value. V rows of kv_b_proj are untouched.

    Returns (w_q_b' , w_kv_b', clipped mask [H] bool, gamma [H]) in float64.
    """
    d = _dims(dims)
    H, N, V, S_ = d.heads, d.nope_dim, d.v_dim, d.shared_dim
    D = N + S_
    wq = np.array(w_q_b, dtype=f64, copy=True)
    wk = np.array(w_kv_b, dtype=f64, copy=True)
    sm = np.asarray(max_logit, dtype=f64)
    mask = sm > tau
    gamma = np.where(mask, tau / np.where(mask, sm, 1.0), 1.0)
    for h in np.nonzero(mask)[0]:
        g = gamma[h]
        r = math.sqrt(g)
        wq[h * D:h * D + N, :] *= r            # q^C rows
        wq[h * D + N:(h + 1) * D, :] *= g      # q^R rows
        wk[h * (N + V):h * (N + V) + N, :] *= r  # K^C rows (W_UK_h)
    return wq, wk, mask, gamma


BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127   # largest finite bf16 value
BF16_MIN_NORMAL = 2.0 ** -126                # bf16 keeps fp32's exponent range
BF16_SUBNORMAL_STEP = 2.0 ** -133            # spacing of bf16 values below the smallest normal


def round_to(x, dtype: str):
    """Round float64 values to the nearest 'f32' or 'bf16' value, ties to even.

    bf16 is fp32's sign and 8 exponent bits with 7 stored fraction bits: 8
    significant bits for normal values, a fixed spacing of 2^-133 below the
    smallest normal 2^-126 (subnormals), and values whose rounding would pass
    the largest finite value (2 - 2^-7) 2^127 become infinite. NaN stays NaN.
    """
    x = np.asarray(x, dtype=f64)
    if dtype == "f32":
        return x.astype(np.float32).astype(f64)
    if dtype != "bf16":
        raise ValueError(dtype)
    with np.errstate(invalid="ignore", over="ignore"):
        m, e = np.frexp(x)                       # x = m * 2^e, 0.5 <= |m| < 1
        r = np.ldexp(np.rint(m * 256.0), e - 8)  # 8 significant bits, half to even
        sub = np.abs(x) < BF16_MIN_NORMAL
        r = np.where(sub, np.rint(x / BF16_SUBNORMAL_STEP) * BF16_SUBNORMAL_STEP, r)
        r = np.where(np.isfinite(r) & (np.abs(r) > BF16_MAX), np.copysign(np.inf, x), r)
    return r
