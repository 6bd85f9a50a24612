"""CPU oracle for gated no-position MLA, its per-head max logit and QK-Clip.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. The product path (the HIP library
and its Python binding) never calls it, and this package imports nothing from
the product.

Everything here is plain NumPy in float64, written from the equations of the
"Kimi K3 · Gated MLA" page (the 20-step equation list and the
``eager_attention_forward`` excerpt) and from the QK-Clip description on the
"SOTA-131" practice page. See ``mla_oracle`` for the functions and which
passage each one follows.
"""
from .mla_oracle import (  # noqa: F401
    Dims,
    absorbed,
    absorbed_max_logit,
    absorbed_rows_selected,
    dense_prefill,
    expand_latent,
    expanded,
    expanded_cache,
    layer_forward,
    layer_rows,
    linear,
    max_logit_head,
    prefill,
    prefill_backward,
    prefill_rows,
    q_projection,
    qk_clip,
    qk_norm_absorbed,
    qk_norm_logit_bound,
    qk_norm_prefill,
    qk_norm_query,
    rms_norm,
    round_to,
)
