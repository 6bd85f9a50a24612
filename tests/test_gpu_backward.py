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
    cu = dev_i32(p.cu_seqlens)
    log(f"backward T={p.ntok} H={dims.heads} seqs={len(p.cu_seqlens) - 1} gate={p.gate is not None}: forward")
    out, lse, _ = m.mla_prefill(ld, q, ckv, ks, w, g, cu, out_dtype=torch.float32, want_lse=True)
    log("backward")
    grads = m.mla_prefill_backward(ld, q, ckv, ks, w, g, cu, out, lse, dev(dout, False))
    torch.cuda.synchronize()
    log("oracle")
    ref = oracle.prefill_backward(p.q, p.ckv, p.ks, p.w_kv_b, p.gate, p.cu_seqlens, dims, dout)
    for name, got, want in zip(["dq", "dckv", "dks", "dw_kv_b", "dgate"], grads, ref):
        if want is None:
            assert got is None
            continue
        got = host(got)
        assert np.isfinite(got).all(), name
        err = rel_err(got, want)
        log(f"  {name}: rel err {err:.3e}")
        assert err <= GRAD_TOL, (name, err)


@pytest.mark.parametrize("gate", [True, False])
def test_backward_ragged_varlen(lib, gate):
    """Two sequences (70 and 129 tokens: not multiples of the 64-row tiles or
    128-row blocks), four heads."""
    p = synth.prefill_inputs(synth.Dims(4, 512, 64, 128, 128), [70, 129], seed=71, bf16=True, gate=gate)
    _check(p, 72)


def test_backward_many_lengths(lib):
    """Ten sequences around every tile and block boundary (1, 31, 32, 63, 64,
    65, 127, 128, 129 tokens) and one of 700 tokens, packed: the work items of
    different sequences interleave in the longest-first order."""
    p = synth.prefill_inputs(synth.Dims(3, 512, 64, 128, 128), [129, 1, 31, 700, 32, 63, 64, 65, 127, 128],
                             seed=78, bf16=True)
    _check(p, 79)


@pytest.mark.parametrize("nseq", [600, 5000])
def test_backward_many_short_sequences(lib, nseq):
    """Hundreds to thousands of packed sequences of 0 to 6 tokens (empty ones
    included) around a 300- and a 129-token one: the plan's counting sort
    lists thousands of one-block work items behind the long ones."""
    rng = np.random.default_rng(nseq)
    lens = [int(x) for x in rng.integers(0, 7, nseq)]
    lens[7], lens[nseq - 10] = 300, 129
    p = synth.prefill_inputs(synth.Dims(2, 512, 64, 128, 128), lens, seed=83, bf16=True)
    _check(p, 84)


def test_backward_96_heads_2048(lib):
    """96 heads, one sequence of 2048 tokens."""
    p = synth.prefill_inputs(synth.K3, [2048], seed=73, bf16=True)
    _check(p, 74)


def test_backward_k3_prefill_4096(lib):
    """The configuration the benchmark times: the Kimi K3 prefill workload
    (T = 4096, 96 heads, gate on), every gradient against the full oracle."""
    _check(synth.k3_prefill(), 75)


def test_backward_16k_sequence(lib):
    """One sequence of 16384 tokens (two heads, so that the fp64 oracle's
    16384 x 16384 planes stay within seconds): 256 query and key tiles per
    head, the longest work items of the plan."""
    p = synth.prefill_inputs(synth.Dims(2, 512, 64, 128, 128), [16384], seed=80, bf16=True)
    _check(p, 81)


def test_backward_empty_and_single_token_sequences(lib):
    """cu_seqlens with a zero-length sequence, a one-token sequence and a
    sequence one row past a 128-row block boundary."""
    p = synth.prefill_inputs(synth.Dims(2, 512, 64, 128, 128), [0, 1, 129], seed=76, bf16=True)
    _check(p, 77)


def test_backward_rejects_host_cu_seqlens(lib):
    """cu_seqlens is read on the device: a host tensor is refused."""
    import torch
    import mla_qk_clip_amd as m
    from tests._gpu import dev, lib_dims
    p = synth.prefill_inputs(synth.Dims(2, 512, 64, 128, 128), [5], seed=82, bf16=True)
    ld = lib_dims(p.dims)
    T, H = p.ntok, p.dims.heads
    with pytest.raises(ValueError):
        m.mla_prefill_backward(ld, dev(p.q, True), dev(p.ckv, True), dev(p.ks, True), dev(p.w_kv_b, True),
                               dev(p.gate, True), torch.from_numpy(p.cu_seqlens), torch.zeros((T, H * 128)).cuda(),
                               torch.zeros((H, T)).cuda(), torch.zeros((T, H * 128)).cuda())
