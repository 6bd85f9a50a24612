"""Seeded synthetic inputs for gated, no-position MLA.

This module only draws random numbers and lays them out. It holds none of the
attention arithmetic, so both the CPU oracle (``oracle/``) and the HIP path
(``mla_qk_clip_amd``) can take their inputs from it without sharing any code
with each other.

Shapes follow the Kimi K3 gated MLA block (96 heads, latent width 512, shared
key width 64, nope width 128, value width 128; "Kimi K3 · Gated MLA" page,
parameter table and the ``KimiMLAAttention`` constructor excerpt).

Value recipe (one reading of "i.i.d. N(0,1)/sqrt(fan_in)"):
  * weights are N(0,1)/sqrt(contracted width): kv_b_proj.weight / sqrt(R),
    q_b_proj.weight / sqrt(q_in);
  * activations (q, c^KV, k^S, c^Q, gate logits g) are N(0,1), i.e. unit RMS,
    as an RMSNorm or a fan-in-scaled projection yields.
With this recipe an unscaled head's logit (after the 1/sqrt(192) factor) has
unit standard deviation, and a head whose q and k weights are multiplied by 40
reaches logits in the thousands.

Draws come from ``numpy.random.default_rng`` (PCG64). Floating-point draws are
float32 ``standard_normal``; bf16 inputs are then rounded to nearest-even.

Layouts (row-major):
  q        [Ntok, H, D]      D = N + S; per head the first N are q^C, the last S are q^R
  ckv      [Ntok, R]         post-RMSNorm latent c^KV
  ks       [Ntok, S]         shared key part k^S (one per token, used by every head)
  w_kv_b   [H*(N+V), R]      kv_b_proj.weight (nn.Linear layout, out x in);
                             head h owns rows h*(N+V) .. : first N rows -> K^C_h, next V -> V_h
  gate     [Ntok, H*V]       gate logits g (sigmoid applied by the method)
  cq       [Ntok, q_in]      post-RMSNorm query latent c^Q (QK-Clip workload only)
  w_q_b    [H*D, q_in]       q_b_proj.weight; head h owns rows h*D .. h*D+D-1
  cache    [B, cap, R+S]     rows [c^KV | k^S]
  lens     [B] int32
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# --------------------------------------------------------------------------
# bf16 helpers (storage format only)
# --------------------------------------------------------------------------


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value (ties to even).

    Returns float32 values that are exactly representable in bf16. NaN stays NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    out = (r & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.float32)
    nan = np.isnan(x)
    if nan.any():
        out = out.copy()
        out[nan] = np.float32("nan")
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns of float32 values that are already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# Dimensions
# --------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class Dims:
    heads: int
    kv_rank: int      # R, width of c^KV
    shared_dim: int   # S, width of k^S / q^R
    nope_dim: int     # N, width of q^C / K^C
    v_dim: int        # V

    @property
    def qk_dim(self) -> int:
        return self.nope_dim + self.shared_dim


K3 = Dims(heads=96, kv_rank=512, shared_dim=64, nope_dim=128, v_dim=128)
TINY = Dims(heads=4, kv_rank=32, shared_dim=16, nope_dim=32, v_dim=32)
K3_Q_LORA_RANK = 1536
CLIP_HEADS = (0, 19, 38, 57, 76, 95)
CLIP_FACTOR = 40.0
TAU = 100.0


def _normal(rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def _quant(x: np.ndarray, bf16: bool) -> np.ndarray:
    return round_bf16(x) if bf16 else np.ascontiguousarray(x, dtype=np.float32)


# --------------------------------------------------------------------------
# Prefill (training-form) inputs
# --------------------------------------------------------------------------


@dataclasses.dataclass
class PrefillInputs:
    dims: Dims
    cu_seqlens: np.ndarray   # int32 [nseq+1]
    q: np.ndarray            # float32 [Ntok, H, D] (bf16-exact when bf16)
    ckv: np.ndarray          # [Ntok, R]
    ks: np.ndarray           # [Ntok, S]
    w_kv_b: np.ndarray       # [H*(N+V), R]
    gate: np.ndarray | None  # [Ntok, H*V]
    bf16: bool
    cq: np.ndarray | None = None     # [Ntok, q_in] (QK-Clip workload)
    w_q_b: np.ndarray | None = None  # [H*D, q_in]  (QK-Clip workload)

    @property
    def ntok(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def max_seqlen(self) -> int:
        return int(np.max(np.diff(self.cu_seqlens))) if len(self.cu_seqlens) > 1 else 0


def prefill_inputs(dims: Dims, seqlens, seed: int, bf16: bool, gate: bool = True) -> PrefillInputs:
    """Draw order: q, c^KV, k^S, kv_b_proj.weight, g."""
    seqlens = [int(x) for x in seqlens]
    cu = np.zeros(len(seqlens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(seqlens)
    n = int(cu[-1])
    H, R, S, N, V = dims.heads, dims.kv_rank, dims.shared_dim, dims.nope_dim, dims.v_dim
    rng = np.random.default_rng(seed)
    q = _quant(_normal(rng, (n, H, N + S)), bf16)
    ckv = _quant(_normal(rng, (n, R)), bf16)
    ks = _quant(_normal(rng, (n, S)), bf16)
    w = _quant(_normal(rng, (H * (N + V), R), 1.0 / math.sqrt(R)), bf16)
    g = _quant(_normal(rng, (n, H * V)), bf16) if gate else None
    return PrefillInputs(dims, cu, q, ckv, ks, w, g, bf16)


def clip_stress_inputs(dims: Dims, seqlen: int, seed: int, q_in: int = K3_Q_LORA_RANK,
                       heads=CLIP_HEADS, factor: float = CLIP_FACTOR) -> PrefillInputs:
    """QK-Clip stress workload (bf16).

    Draw order: c^Q, q_b_proj.weight, c^KV, k^S, kv_b_proj.weight, g. In the
    listed heads every q_b_proj row of the head (all D columns of W_UQ's head
    block) and the N K^C rows of kv_b_proj (not the V rows) are multiplied by
    ``factor`` before bf16 rounding. ``q`` is left as None: the query
    projection belongs to the caller (q = c^Q W_UQ).
    """
    H, R, S, N, V = dims.heads, dims.kv_rank, dims.shared_dim, dims.nope_dim, dims.v_dim
    D = N + S
    n = int(seqlen)
    rng = np.random.default_rng(seed)
    cq = round_bf16(_normal(rng, (n, q_in)))
    wq = _normal(rng, (H * D, q_in), 1.0 / math.sqrt(q_in))
    ckv = round_bf16(_normal(rng, (n, R)))
    ks = round_bf16(_normal(rng, (n, S)))
    w = _normal(rng, (H * (N + V), R), 1.0 / math.sqrt(R))
    g = round_bf16(_normal(rng, (n, H * V)))
    for h in heads:
        wq[h * D:(h + 1) * D, :] *= np.float32(factor)
        w[h * (N + V):h * (N + V) + N, :] *= np.float32(factor)
    cu = np.array([0, n], dtype=np.int32)
    return PrefillInputs(dims, cu, None, ckv, ks, round_bf16(w), g, True,
                         cq=cq, w_q_b=round_bf16(wq))


# --------------------------------------------------------------------------
# Whole-layer inputs (x and every projection of the attention layer)
# --------------------------------------------------------------------------

K3_HIDDEN = 7168


@dataclasses.dataclass
class LayerInputs:
    dims: Dims
    hidden: int
    q_rank: int
    cu_seqlens: np.ndarray   # int32 [nseq+1]
    x: np.ndarray            # [Ntok, hidden]
    w_dq: np.ndarray         # q_a_proj.weight [q_rank, hidden]
    g_q: np.ndarray          # q_a_layernorm.weight [q_rank]
    w_uq: np.ndarray         # q_b_proj.weight [H*D, q_rank]
    w_kv_a: np.ndarray       # kv_a_proj_with_mqa.weight [R+S, hidden]
    g_kv: np.ndarray         # kv_a_layernorm.weight [R]
    w_kv_b: np.ndarray       # kv_b_proj.weight [H*(N+V), R]
    w_g: np.ndarray          # g_proj.weight [H*V, hidden]
    w_o: np.ndarray          # o_proj.weight [hidden, H*V]
    bf16: bool

    @property
    def ntok(self) -> int:
        return int(self.cu_seqlens[-1])


def layer_inputs(dims: Dims, hidden: int, q_rank: int, seqlens, seed: int, bf16: bool = True) -> LayerInputs:
    """Draw order: x, w_dq, g_q, w_uq, w_kv_a, g_kv, w_kv_b, w_g, w_o.

    x ~ N(0,1); every projection N(0,1)/sqrt(fan_in); RMSNorm weights
    1 + 0.1 N(0,1) (trained norms sit near their initial 1).
    """
    H, R, S, N, V = dims.heads, dims.kv_rank, dims.shared_dim, dims.nope_dim, dims.v_dim
    D = N + S
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32)
    n = int(cu[-1])
    x = _quant(_normal(rng, (n, hidden)), bf16)
    w_dq = _quant(_normal(rng, (q_rank, hidden), 1.0 / math.sqrt(hidden)), bf16)
    g_q = _quant(1.0 + _normal(rng, (q_rank,), 0.1), bf16)
    w_uq = _quant(_normal(rng, (H * D, q_rank), 1.0 / math.sqrt(q_rank)), bf16)
    w_kv_a = _quant(_normal(rng, (R + S, hidden), 1.0 / math.sqrt(hidden)), bf16)
    g_kv = _quant(1.0 + _normal(rng, (R,), 0.1), bf16)
    w_kv_b = _quant(_normal(rng, (H * (N + V), R), 1.0 / math.sqrt(R)), bf16)
    w_g = _quant(_normal(rng, (H * V, hidden), 1.0 / math.sqrt(hidden)), bf16)
    w_o = _quant(_normal(rng, (hidden, H * V), 1.0 / math.sqrt(H * V)), bf16)
    return LayerInputs(dims, hidden, q_rank, cu, x, w_dq, g_q, w_uq, w_kv_a, g_kv, w_kv_b, w_g, w_o, bf16)


# --------------------------------------------------------------------------
# Absorbed-form (decode) inputs
# --------------------------------------------------------------------------


@dataclasses.dataclass
class DecodeInputs:
    dims: Dims
    lens: np.ndarray          # int32 [B]
    cap: int                  # rows allocated per sequence
    tq: int                   # query tokens per sequence
    q: np.ndarray             # [B, Tq, H, D]
    w_kv_b: np.ndarray        # [H*(N+V), R]
    gate: np.ndarray | None   # [B, Tq, H*V]
    bf16: bool
    seed: int

    @property
    def batch(self) -> int:
        return int(self.lens.shape[0])

    @property
    def max_len(self) -> int:
        return int(self.lens.max()) if self.lens.size else 0

    def cache_rows(self, b: int) -> np.ndarray:
        """The lens[b] valid rows [c^KV | k^S] of sequence b, float32 [lens[b], R+S].

        Each sequence has its own child stream (spawned from the workload
        seed), so any subset of sequences can be drawn without drawing the rest.
        """
        child = np.random.SeedSequence(self.seed).spawn(self.batch)[b]
        rng = np.random.default_rng(child)
        rows = _normal(rng, (int(self.lens[b]), self.dims.kv_rank + self.dims.shared_dim))
        return _quant(rows, self.bf16)


def decode_inputs(dims: Dims, lens, cap: int, tq: int, seed: int, bf16: bool,
                  gate: bool = True) -> DecodeInputs:
    """Draw order: q, kv_b_proj.weight, g; cache rows per sequence from child streams."""
    lens = np.asarray(lens, dtype=np.int32)
    B = lens.shape[0]
    H, R, S, N, V = dims.heads, dims.kv_rank, dims.shared_dim, dims.nope_dim, dims.v_dim
    rng = np.random.default_rng(seed)
    q = _quant(_normal(rng, (B, tq, H, N + S)), bf16)
    w = _quant(_normal(rng, (H * (N + V), R), 1.0 / math.sqrt(R)), bf16)
    g = _quant(_normal(rng, (B, tq, H * V)), bf16) if gate else None
    return DecodeInputs(dims, lens, int(cap), int(tq), q, w, g, bf16, seed)


def expanded_rows(dims: Dims, L: int, seed: int, b: int = 0, bf16: bool = True):
    """Per-head cache rows of one sequence for the expanded-cache decode:
    K [H, L, N+S] and V [H, L, V], N(0,1) entries (the spread of K^C = c^KV W_UK,
    k^S and V under the weight recipe), rounded to bf16; float32.

    Sequence b draws from its own child stream of ``seed``.
    """
    rng = np.random.default_rng(np.random.SeedSequence([seed, 13, b]))
    H, D, V = dims.heads, dims.nope_dim + dims.shared_dim, dims.v_dim
    k = _quant(_normal(rng, (H, L, D)), bf16)
    v = _quant(_normal(rng, (H, L, V)), bf16)
    return k, v


def decode_lens(batch: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Per-sequence cache lengths, uniform integers in [lo, hi]."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 7]))
    return rng.integers(lo, hi, size=batch, endpoint=True).astype(np.int32)


# --------------------------------------------------------------------------
# The five named workloads
# --------------------------------------------------------------------------

VARLEN_SEQLENS = (32768, 16384, 8192, 2048)


def tiny_fp32_prefill(seed: int = 0) -> PrefillInputs:
    """Tiny fp32 case: B=1, T=64, H=4, R=32, S=16, N=V=32."""
    return prefill_inputs(TINY, [64], seed, bf16=False)


def tiny_fp32_absorbed(seed: int = 0):
    """The tiny case as an absorbed call: Tq=64 queries over a 64-row cache.

    The cache rows are the same c^KV and k^S values as ``tiny_fp32_prefill``.
    Returns (prefill inputs, q [1,64,H,D], cache [1,64,R+S], lens [1], gate [1,64,H*V]).
    """
    p = tiny_fp32_prefill(seed)
    cache = np.concatenate([p.ckv, p.ks], axis=1)[None]
    return p, p.q[None], cache, np.array([64], dtype=np.int32), p.gate[None]


def k3_prefill(seed: int = 1, seqlen: int = 4096) -> PrefillInputs:
    """K3-shaped gated prefill: B=1, T=4096, bf16."""
    return prefill_inputs(K3, [seqlen], seed, bf16=True)


def k3_decode(seed: int = 2, batch: int = 64, cap: int = 32768, lo: int = 1024) -> DecodeInputs:
    """Absorbed decode: 64 sequences, one query each, cache rows <= 32768, bf16."""
    lens = decode_lens(batch, lo, cap, seed)
    return decode_inputs(K3, lens, cap, 1, seed, bf16=True)


def k3_clip_stress(seed: int = 3, seqlen: int = 2048) -> PrefillInputs:
    """QK-Clip stress: as the K3 prefill with T=2048 and six heads scaled x40."""
    return clip_stress_inputs(K3, seqlen, seed)


def k3_varlen(seed: int = 4, seqlens=VARLEN_SEQLENS) -> PrefillInputs:
    """Long-context packed varlen prefill: 32768 + 16384 + 8192 + 2048 tokens."""
    return prefill_inputs(K3, list(seqlens), seed, bf16=True)


def k3_layer(seed: int = 5, seqlen: int = 4096) -> LayerInputs:
    """The whole Kimi K3 attention layer (hidden 7168, q_lora_rank 1536) at T = seqlen."""
    return layer_inputs(K3, K3_HIDDEN, K3_Q_LORA_RANK, [seqlen], seed, bf16=True)


def k3_q_weight(seed: int = 11, q_in: int = K3_Q_LORA_RANK) -> np.ndarray:
    """q_b_proj.weight [96*192, 1536] ~ N(0,1)/sqrt(1536), bf16 (for a clip step without clipped heads)."""
    rng = np.random.default_rng(seed)
    return round_bf16(_normal(rng, (K3.heads * K3.qk_dim, q_in), 1.0 / math.sqrt(q_in)))
