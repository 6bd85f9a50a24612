"""GPU-test helpers: upload seeded inputs, call the library, compare."""
import sys
import time

import numpy as np
import torch

import synth


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def dev(x, bf16: bool):
    """float32 numpy array (bf16-exact when bf16) -> contiguous device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    return t.to(torch.bfloat16) if bf16 else t


def dev_i32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def lib_dims(d):
    import mla_qk_clip_amd as m
    return m.Dims(d.heads, d.kv_rank, d.shared_dim, d.nope_dim, d.v_dim)


def run_prefill(p: synth.PrefillInputs, q=None, out_dtype=torch.float32, want_lse=True, max_logit=None,
                accumulate=False):
    import mla_qk_clip_amd as m
    q = p.q if q is None else q
    bf = p.bf16
    out, lse, ml = m.mla_prefill(lib_dims(p.dims), dev(q, bf), dev(p.ckv, bf), dev(p.ks, bf), dev(p.w_kv_b, bf),
                                 None if p.gate is None else dev(p.gate, bf), dev_i32(p.cu_seqlens),
                                 out_dtype=out_dtype, want_lse=want_lse, max_logit=max_logit,
                                 accumulate=accumulate)
    torch.cuda.synchronize()
    return out, lse, ml


def decode_cache_tensor(d: synth.DecodeInputs, poison=True):
    """Device cache [B, cap, R+S]; rows at or past lens[b] hold NaN (poison)."""
    W = d.dims.kv_rank + d.dims.shared_dim
    dt = torch.bfloat16 if d.bf16 else torch.float32
    fill = float("nan") if poison else 0.0
    cache = torch.full((d.batch, d.cap, W), fill, dtype=dt, device="cuda")
    for b in range(d.batch):
        rows = d.cache_rows(b)
        cache[b, :rows.shape[0]] = dev(rows, d.bf16)
    return cache


def run_absorbed(d: synth.DecodeInputs, cache=None, out_dtype=None, max_logit=None, accumulate=False):
    import mla_qk_clip_amd as m
    cache = decode_cache_tensor(d) if cache is None else cache
    out, ml = m.mla_absorbed(lib_dims(d.dims), dev(d.q, d.bf16), cache, dev_i32(d.lens), dev(d.w_kv_b, d.bf16),
                             None if d.gate is None else dev(d.gate, d.bf16), out_dtype=out_dtype,
                             max_logit=max_logit, accumulate=accumulate)
    torch.cuda.synchronize()
    return out, ml
