"""The no-allocation absorbed entry point, mla_absorbed_noalloc, against the
workspace entry point mla_absorbed: the same kernels with their scratch memory
in the library's static device array, so the outputs and max logits must be
bit-for-bit those of mla_absorbed. Two calls in a row, the second smaller than
the first, so the second runs on the scratch contents the first left behind.
"""
import numpy as np
import pytest

import oracle
import synth
from tests._util import rel_err

pytestmark = pytest.mark.gpu


def _inputs(d):
    from tests._gpu import decode_cache_tensor, dev, dev_i32
    return (dev(d.q, True), decode_cache_tensor(d), dev_i32(d.lens), dev(d.w_kv_b, True),
            None if d.gate is None else dev(d.gate, True))


@pytest.mark.parametrize("out_f32", [False, True])
def test_noalloc_matches_workspace_entry_point_on_two_calls(gpu_available, out_f32):
    import torch
    import mla_qk_clip_amd as m
    from tests._gpu import host, lib_dims, log
    dt = torch.float32 if out_f32 else torch.bfloat16
    big = synth.decode_inputs(synth.K3, [3000, 1200, 5, 2500, 64], cap=3008, tq=2, seed=51, bf16=True)
    small = synth.decode_inputs(synth.K3, [700, 33], cap=704, tq=1, seed=52, bf16=True)
    dims = lib_dims(synth.K3)
    runs = []
    for d in (big, small):
        q, cache, lens, w, g = _inputs(d)
        out = torch.empty((d.batch, d.tq, 96 * 128), dtype=dt, device="cuda")
        ml = torch.empty(96, dtype=torch.float32, device="cuda")
        runs.append((d, (q, cache, lens, w, g), out, ml))
    log(f"no-alloc absorbed: two calls in a row (fp32 out={out_f32})")
    for d, (q, cache, lens, w, g), out, ml in runs:
        m.mla_absorbed_noalloc(dims, q, cache, lens, w, g, out=out, max_logit=ml)
    torch.cuda.synchronize()
    log("workspace entry point on the same inputs")
    for d, (q, cache, lens, w, g), out, ml in runs:
        ref_out, ref_ml = m.mla_absorbed(dims, q, cache, lens, w, g, out_dtype=dt)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out)
        assert torch.equal(ml, ref_ml)
    # and the smaller call against the oracle, at the library's tolerances
    d = small
    rows = [d.cache_rows(b) for b in range(d.batch)]
    ref, ref_sm = oracle.absorbed(d.q, rows, d.w_kv_b, d.gate, d.dims)
    assert rel_err(host(runs[1][2]), ref) <= 2e-2
    assert np.all(np.abs(host(runs[1][3]) - ref_sm) / np.abs(ref_sm) <= 1e-3)


def test_noalloc_accumulates_and_rejects_sizes_past_its_scratch(gpu_available):
    import torch
    import mla_qk_clip_amd as m
    from tests._gpu import lib_dims, log
    d = synth.decode_inputs(synth.K3, [900, 400], cap=904, tq=1, seed=53, bf16=True)
    dims = lib_dims(synth.K3)
    q, cache, lens, w, g = _inputs(d)
    out = torch.empty((d.batch, 1, 96 * 128), dtype=torch.bfloat16, device="cuda")
    ml = torch.full((96,), 1e4, dtype=torch.float32, device="cuda")
    log("no-alloc absorbed: accumulate into a preset max logit")
    m.mla_absorbed_noalloc(dims, q, cache, lens, w, g, out=out, max_logit=ml, accumulate=True)
    torch.cuda.synchronize()
    assert bool((ml == 1e4).all())
    _, alone = m.mla_absorbed(dims, q, cache, lens, w, g)
    m.mla_absorbed_noalloc(dims, q, cache, lens, w, g, out=out, max_logit=ml)
    torch.cuda.synchronize()
    assert torch.equal(ml, alone)
    # 256 single-token sequences need more than the built-in 128 MiB: refused before any launch
    B = 256
    qb = torch.zeros((B, 1, 96, 192), dtype=torch.bfloat16, device="cuda")
    cb = torch.zeros((B, 8, 576), dtype=torch.bfloat16, device="cuda")
    lb = torch.full((B,), 8, dtype=torch.int32, device="cuda")
    ob = torch.empty((B, 1, 96 * 128), dtype=torch.bfloat16, device="cuda")
    assert m.mla_absorbed_workspace_size(dims, m.MLA_BF16, B, 1) > 128 << 20
    with pytest.raises(m.MlaError, match="built-in scratch"):
        m.mla_absorbed_noalloc(dims, qb, cb, lb, w, None, out=ob, max_logit=ml)
