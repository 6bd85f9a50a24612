"""GPU parity of the prefill backward (mla_prefill_backward) against the CPU oracle."""
import numpy as np
import pytest

import oracle
import synth
from tests._util import rel_err

pytestmark = pytest.mark.gpu

GRAD_TOL = 2e-2


@pytest.fixture(scope="module")
def lib(gpu_available):
    import mla_qk_clip_amd as m
    return m


def _check(p, seed):
    import torch
    import mla_qk_clip_amd as m
    from tests._gpu import dev, dev_i32, host, lib_dims, log
    dims = p.dims
    rng = np.random.default_rng(seed)
    dout = rng.standard_normal((p.ntok, dims.heads * dims.v_dim)).astype(np.float32)
    ld = lib_dims(dims)
    q, ckv, ks, w = dev(p.q, True), dev(p.ckv, True), dev(p.ks, True), dev(p.w_kv_b, True)
    g = None if p.gate is None else dev(p.gate, True)
    log(f"backward T={p.ntok} H={dims.heads} gate={p.gate is not None}: forward")
    out, lse, _ = m.mla_prefill(ld, q, ckv, ks, w, g, dev_i32(p.cu_seqlens), out_dtype=torch.float32, want_lse=True)
    log("backward")
    grads = m.mla_prefill_backward(ld, q, ckv, ks, w, g, p.cu_seqlens, out, lse, dev(dout, False))
    torch.cuda.synchronize()
    log("oracle")
    ref = oracle.prefill_backward(p.q, p.ckv, p.ks, p.w_kv_b, p.gate, p.cu_seqlens, dims, dout)
    for name, got, want in zip(["dq", "dckv", "dks", "dw_kv_b", "dgate"], grads, ref):
        if want is None:
            assert got is None
            continue
        err = rel_err(host(got), want)
        log(f"  {name}: rel err {err:.3e}")
        assert err <= GRAD_TOL, (name, err)


@pytest.mark.parametrize("gate", [True, False])
def test_backward_ragged_varlen(lib, gate):
    """Two sequences (70 and 129 tokens: not multiples of the 128-row padding),
    four heads."""
    p = synth.prefill_inputs(synth.Dims(4, 512, 64, 128, 128), [70, 129], seed=71, bf16=True, gate=gate)
    _check(p, 72)


def test_backward_96_heads_2048(lib):
    """96 heads, one sequence of 2048 tokens (12 chunks of 8 heads)."""
    p = synth.prefill_inputs(synth.K3, [2048], seed=73, bf16=True)
    _check(p, 74)


def test_backward_k3_prefill_4096(lib):
    """The configuration the benchmark times: the Kimi K3 prefill workload
    (T = 4096, 96 heads, gate on), every gradient against the full oracle."""
    _check(synth.k3_prefill(), 75)


def test_backward_empty_and_single_token_sequences(lib):
    """cu_seqlens with a zero-length sequence, a one-token sequence and a
    sequence one row past a 128-row padding boundary."""
    p = synth.prefill_inputs(synth.Dims(2, 512, 64, 128, 128), [0, 1, 129], seed=76, bf16=True)
    _check(p, 77)
