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


@pytest.mark.parametrize("heads", [20, 128])
def test_bf16_decode_other_head_counts(lib, heads):
    """Head counts other than 96: 20 (one partial block of 32 heads in the
    split workgroups' single row) and 128 (the largest supported: a second row
    of split workgroups holding 32 heads). Nine ragged sequences with two query
    tokens each give 18 virtual sequences, so the finishing kernel's last
    combine block is partial."""
    from tests._gpu import host, log, run_absorbed
    dims = synth.Dims(heads=heads, kv_rank=512, shared_dim=64, nope_dim=128, v_dim=128)
    d = synth.decode_inputs(dims, [5, 700, 33, 2100, 64, 2, 900, 31, 4097], cap=4104, tq=2, seed=41, bf16=True)
    log(f"bf16 absorbed heads={heads} batch=9 tq=2")
    out, ml = run_absorbed(d)
    rows = [d.cache_rows(b) for b in range(d.batch)]
    ref, ref_sm = oracle.absorbed(d.q, rows, d.w_kv_b, d.gate, d.dims)
    assert rel_err(host(out), ref) <= BF16_TOL
    assert np.all(np.abs(host(ml) - ref_sm) / np.abs(ref_sm) <= SMAX_TOL)


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


@pytest.mark.parametrize("tq", [1, 2])
def test_bf16_decode_fewer_rows_than_splits(lib, tq):
    """Fewer visible cache rows in total than split workgroups: some splits
    hold no rows and write no partial, and the merge must skip them."""
    from tests._gpu import host, log, run_absorbed
    d = synth.decode_inputs(synth.K3, [5, 33, 2, 17], cap=64, tq=tq, seed=35, bf16=True)
    log(f"bf16 absorbed, {int(d.lens.sum())} rows in total, tq={tq}")
    out, ml = run_absorbed(d)
    rows = [d.cache_rows(b) for b in range(d.batch)]
    ref, ref_sm = oracle.absorbed(d.q, rows, d.w_kv_b, d.gate, d.dims)
    assert rel_err(host(out), ref) <= BF16_TOL
    # with a few dozen rows the largest logit sits only ~2 sigma out, where
    # the bf16 rounding of q_abs alone would exceed 1e-3 relative: the
    # refinement re-scores the candidate tiles in fp32
    assert np.all(np.abs(host(ml) - ref_sm) / np.abs(ref_sm) <= SMAX_TOL)


@pytest.mark.parametrize("tq", [1, 2])
def test_bf16_decode_more_sequences_than_splits(lib, tq):
    """700 sequences, far more than the 256 split workgroups: most hold tq to
    40 rows, so a split's row range covers many whole sequences (cuts snap to
    sequence starts), and three long ones are cut over several splits."""
    from tests._gpu import host, log, run_absorbed
    rng = np.random.default_rng(700 + tq)
    lens = rng.integers(tq, 41, 700).astype(np.int32)
    lens[[3, 350, 699]] = [2900, 1500, 2999]
    d = synth.decode_inputs(synth.K3, lens, cap=3008, tq=tq, seed=36, bf16=True)
    log(f"bf16 absorbed, {d.batch} sequences, {int(lens.sum())} rows, tq={tq}")
    out, ml = run_absorbed(d)
    rows = [d.cache_rows(b) for b in range(d.batch)]
    ref, ref_sm = oracle.absorbed(d.q, rows, d.w_kv_b, d.gate, d.dims)
    assert rel_err(host(out), ref) <= BF16_TOL
    assert np.all(np.abs(host(ml) - ref_sm) / np.abs(ref_sm) <= SMAX_TOL)


def test_bf16_decode_max_logit_init_and_accumulate(lib):
    """Without accumulate the max-logit slots are reset (a stale value above
    every logit does not survive); with accumulate the call folds its maxima
    into what the slots hold."""
    import torch
    from tests._gpu import host, log, run_absorbed
    d1 = synth.decode_inputs(synth.K3, [300, 40], cap=320, tq=1, seed=36, bf16=True)
    d2 = synth.decode_inputs(synth.K3, [700], cap=704, tq=1, seed=37, bf16=True)
    log("bf16 absorbed max-logit init / accumulate")
    ml = torch.full((d1.dims.heads,), 1e4, dtype=torch.float32, device="cuda")
    run_absorbed(d1, max_logit=ml)
    ml1 = host(ml).copy()
    rows1 = [d1.cache_rows(b) for b in range(d1.batch)]
    _, ref1 = oracle.absorbed(d1.q, rows1, d1.w_kv_b, d1.gate, d1.dims)
    assert np.all(np.abs(ml1 - ref1) / np.abs(ref1) <= SMAX_TOL)
    _, alone = run_absorbed(d2)
    run_absorbed(d2, max_logit=ml, accumulate=True)
    assert np.array_equal(host(ml), np.maximum(ml1, host(alone)))


def test_bf16_decode_logit_spike_takes_fixup_path(lib):
    """One row deep inside each of two sequences scaled x60: for the heads
    where it scores positively its logit exceeds the first rows' by far more
    than the split kernel's fixed softmax reference allows, so those segments
    are flagged and recomputed by the fix-up kernel; the result still matches
    the oracle. (A single dominant row: near-ties between several huge logits
    would measure the bf16 rounding of q_abs instead.)"""
    import torch
    from tests._gpu import dev, host, log, run_absorbed
    d = synth.decode_inputs(synth.K3, [3000, 2500, 700], cap=3008, tq=1, seed=34, bf16=True)
    rows = [d.cache_rows(b).copy() for b in range(d.batch)]
    rows[0][1500] = synth.round_bf16(rows[0][1500] * 60.0)
    rows[1][2400] = synth.round_bf16(rows[1][2400] * 60.0)
    W = d.dims.kv_rank + d.dims.shared_dim
    cache = torch.full((d.batch, d.cap, W), float("nan"), dtype=torch.bfloat16, device="cuda")
    for b in range(d.batch):
        cache[b, :rows[b].shape[0]] = dev(rows[b], True)
    log("bf16 absorbed with logit spikes")
    out, ml = run_absorbed(d, cache=cache)
    ref, ref_sm = oracle.absorbed(d.q, rows, d.w_kv_b, d.gate, d.dims)
    # the spikes dominate: the largest logits are tens of times the normal ones
    assert ref_sm.max() > 40.0
    assert rel_err(host(out), ref) <= BF16_TOL
    # The streamed logits use q_abs rounded to bf16; at logits this large
    # their error exceeds 1e-3 relative, and the refined max logit does not.
    assert np.all(np.abs(host(ml) - ref_sm) / np.abs(ref_sm) <= SMAX_TOL)


@pytest.mark.parametrize("tq", [1, 2])
def test_bf16_decode_max_logit_exact_on_ties(lib, tq):
    """Every row of a long sequence identical: every tile of each head is a
    candidate, more than a refine workgroup lists, so the refinement re-scores
    the split workgroups' candidate tiles directly and the max logit is still
    exact (to 1e-3); the second sequence (ordinary rows) is unaffected in the
    output. With two query tokens per sequence the virtual sequences see
    different row counts."""
    import torch
    from tests._gpu import dev, host, log, run_absorbed
    d = synth.decode_inputs(synth.K3, [9000, 700], cap=9024, tq=tq, seed=38, bf16=True)
    rows = [d.cache_rows(b).copy() for b in range(d.batch)]
    rows[0][:] = rows[0][0]
    W = d.dims.kv_rank + d.dims.shared_dim
    cache = torch.full((d.batch, d.cap, W), float("nan"), dtype=torch.bfloat16, device="cuda")
    for b in range(d.batch):
        cache[b, :rows[b].shape[0]] = dev(rows[b], True)
    log("bf16 absorbed, 9000 identical rows")
    out, ml = run_absorbed(d, cache=cache)
    ref, ref_sm = oracle.absorbed(d.q, rows, d.w_kv_b, d.gate, d.dims)
    assert rel_err(host(out), ref) <= BF16_TOL
    assert np.all(np.abs(host(ml) - ref_sm) / np.abs(ref_sm) <= SMAX_TOL)


def test_bf16_decode_max_logit_exact_when_every_list_overflows(lib):
    """Sixteen sequences of 20000 identical rows each (one row drawn per
    sequence): every split workgroup holds about 39 tied candidate tiles per
    head, more than its list keeps, so every list overflows and the
    refinement re-scores all rows of every split workgroup. Identical rows
    make the exact references those of one row per sequence: the softmax is
    uniform, the output is the row's value mix and the max logit its logit."""
    import torch
    from tests._gpu import dev, host, log, run_absorbed
    L = 20000
    d = synth.decode_inputs(synth.K3, [L] * 16, cap=L, tq=1, seed=39, bf16=True)
    one = [d.cache_rows(b)[:1].copy() for b in range(d.batch)]
    W = d.dims.kv_rank + d.dims.shared_dim
    cache = torch.empty((d.batch, d.cap, W), dtype=torch.bfloat16, device="cuda")
    for b in range(d.batch):
        cache[b] = dev(one[b], True).expand(L, W)
    log(f"bf16 absorbed, {d.batch} x {L} identical rows")
    out, ml = run_absorbed(d, cache=cache)
    ref, ref_sm = oracle.absorbed(d.q, one, d.w_kv_b, d.gate, d.dims)
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

    class _Rows:   # sequence b's rows, drawn when the oracle asks for them
        def __getitem__(self, b):
            return rows[b] if b in rows else d.cache_rows(b)

    sm = oracle.absorbed_max_logit(d.q, _Rows(), d.w_kv_b, d.dims)
    assert np.all(np.abs(host(ml) - sm) / np.abs(sm) <= SMAX_TOL)


def test_bf16_decode_deterministic(lib):
    from tests._gpu import decode_cache_tensor, log, run_absorbed
    d = synth.decode_inputs(synth.K3, [2000, 777, 1], cap=2048, tq=1, seed=34, bf16=True)
    cache = decode_cache_tensor(d)
    log("decode determinism")
    o1, m1 = run_absorbed(d, cache=cache)
    o2, m2 = run_absorbed(d, cache=cache)
    assert bool((o1 == o2).all()) and bool((m1 == m2).all())
