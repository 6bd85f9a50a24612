"""Benchmark of the gated-MLA hot path on one MI355X.

One step = the whole path on seeded synthetic inputs shaped like Kimi K3's MLA
layers, inputs resident in HBM:
  1. mla_prefill  : training-form gated prefill, B=1, T=4096, H=96, bf16 in,
                    fp32 out, with the fused per-head max logit;
  2. mla_qk_clip  : QK-Clip on q_b_proj / kv_b_proj from that max logit (tau=100);
  3. mla_absorbed : absorbed decode, 64 sequences x 1 query over a latent cache
                    of up to 32768 rows x 576 bf16 per sequence.

``value`` is the prefill's algorithmic TFLOP/s (expansion + QK^T + PV over the
causal pairs) from HIP events around the prefill calls; the decode's cache
GB/s and the per-kernel roofline figures are reported beside it.

Five legs are timed apart from the step and reported in their own objects:
``clip_stress`` (the QK-Clip stress workload at T=2048: the attention pass
before and after a clip that rescales six heads, and the clip), ``layer``
(the whole attention layer at T=4096: projections, RMSNorms, attention,
output projection), ``backward`` (the gradients of the T=4096 prefill),
``varlen_prefill`` (the long packed prefill, 59,392 tokens) and
``expanded_decode`` (the decode workload over a per-head K/V cache, the
comparator of the latent cache).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-decode]
                       [--no-clip-stress] [--no-layer] [--no-backward] [--no-varlen] [--no-expanded]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
METRIC = "MLA prefill TFLOP/s (%MFMA peak); absorbed decode cache GB/s (%HBM peak)"


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def prefill_flops(T: int, H: int, R: int = 512, D: int = 192, V: int = 128):
    pairs = T * (T + 1) // 2
    qk = 2.0 * H * pairs * D
    pv = 2.0 * H * pairs * V
    expand = 2.0 * T * H * 256 * R
    return qk, pv, expand


def source_digest(files) -> str:
    """sha256 over the kernel sources a counter table was taken with."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded(table: str, field: str, files):
    """One figure of a committed rocprofv3 summary (profiles/<table>.md, lines
    "- field: `value`"), or None when the table is missing or the kernel
    sources changed since its counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{table}.md")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as fh:
        for line in fh:
            m = re.match(r"^- (\w+): `?([^`\s]+)`?", line.strip())
            if m:
                rec[m.group(1)] = m.group(2)
    if rec.get("source_sha256") != source_digest(files):
        return None
    try:
        return float(rec[field])
    except (KeyError, ValueError):
        return None


def recorded_traffic(kernel: str, files):
    """HBM bytes per launch of `kernel` (profiles/traffic_<kernel>.md: FETCH_SIZE +
    WRITE_SIZE per dispatch, scaled by the copy-kernel calibration), or None."""
    v = recorded(f"traffic_{kernel}", "bytes_per_launch", files)
    return None if v is None else int(v)


def recorded_mfma_busy(kernel: str, files):
    """Fraction of SIMD cycles the matrix cores were busy during `kernel`
    (profiles/mfma_<kernel>.md: SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE
    per XCD x 1024 SIMDs), or None."""
    return recorded(f"mfma_{kernel}", "mfma_busy", files)


PREFILL_SOURCES = ("mla_qk_clip_amd/csrc/prefill_bf16.hip", "mla_qk_clip_amd/csrc/mla_common.h",
                   "mla_qk_clip_amd/csrc/mla_internal.h")
DECODE_SOURCES = ("mla_qk_clip_amd/csrc/absorbed_bf16.hip", "mla_qk_clip_amd/csrc/mla_common.h",
                  "mla_qk_clip_amd/csrc/mla_internal.h")
EXPANDED_SOURCES = ("mla_qk_clip_amd/csrc/expanded_bf16.hip", "mla_qk_clip_amd/csrc/mla_common.h",
                    "mla_qk_clip_amd/csrc/mla_internal.h")
BACKWARD_SOURCES = ("mla_qk_clip_amd/csrc/backward_bf16.hip", "mla_qk_clip_amd/csrc/mla_common.h",
                    "mla_qk_clip_amd/csrc/mla_internal.h")
LAYER_SOURCES = ("mla_qk_clip_amd/csrc/layer_bf16.hip", "mla_qk_clip_amd/csrc/mla_common.h",
                 "mla_qk_clip_amd/csrc/mla_internal.h")


def cpu_baseline(p, budget_s: float = 12.0):
    """The oracle (fp64 NumPy) on a bounded sample of the same prefill: whole
    heads, one after another, until about ``budget_s`` seconds have passed."""
    import oracle
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        cores = len(os.sched_getaffinity(0))
    T, H = p.ntok, p.dims.heads
    qk, pv, ex = prefill_flops(T, H)
    per_head = (qk + pv + ex) / H
    heads = 0
    t0 = time.perf_counter()
    while heads < H:
        oracle.prefill(p.q, p.ckv, p.ks, p.w_kv_b, p.gate, p.cu_seqlens, p.dims, heads=[heads])
        heads += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": per_head * heads / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{heads} of {H} heads of the T={T} prefill (fp64 NumPy), {dt:.1f} s",
            "cpu": cpu_model(), "cores_available": len(os.sched_getaffinity(0))}


def cpu_model() -> str:
    """The host CPU's model name (first 'model name' line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def varlen_leg(m, dims, steps: int = 3):
    """The long packed prefill: sequences of 32768, 16384, 8192 and 2048 tokens
    (59,392 in all), 96 heads, gate on, fp32 out. Inputs are drawn on the device
    (seeded torch generator) with the synthetic recipe's spreads: N(0,1)
    activations, kv_b_proj N(0,1)/sqrt(512)."""
    import torch
    import synth
    lens = list(synth.VARLEN_SEQLENS)
    T, H = sum(lens), 96
    log(f"long varlen prefill leg ({'+'.join(map(str, lens))} tokens)")
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    bf = dict(generator=g, dtype=torch.bfloat16, device="cuda")
    q = torch.randn((T, H, 192), **bf)
    ckv = torch.randn((T, 512), **bf)
    ks = torch.randn((T, 64), **bf)
    w = (torch.randn((H * 256, 512), generator=g, dtype=torch.float32, device="cuda") / 512 ** 0.5).to(torch.bfloat16)
    gate = torch.randn((T, H * 128), **bf)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
    out = torch.empty((T, H * 128), dtype=torch.float32, device="cuda")
    ml = torch.empty(H, dtype=torch.float32, device="cuda")
    ws = torch.empty(m.mla_prefill_workspace_size(dims, m.MLA_BF16, T, len(lens)), dtype=torch.uint8, device="cuda")

    def call():
        m.mla_prefill(dims, q, ckv, ks, w, gate, cu, out=out, max_logit=ml, workspace=ws)
    call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        call()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    pairs = sum(L * (L + 1) // 2 for L in lens)
    fl = 2.0 * H * pairs * (192 + 128) + 2.0 * T * H * 256 * 512
    del q, ckv, ks, w, gate, out, ws
    torch.cuda.empty_cache()
    return {"workload": "Kimi K3 gated MLA prefill, packed 32768+16384+8192+2048 tokens, H=96, bf16 in, fp32 out",
            "ms": round(ms, 3), "gflop": round(fl / 1e9, 1), "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
            "frac_mfma_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def backward_leg(m, dims, p, q, ckv, ks, w_kv_b, gate, cu, steps: int = 3):
    """Backward of the T=4096 prefill: gradients of q, c^KV, k^S, kv_b_proj
    and the gate for a seeded upstream gradient, from the forward's lse."""
    import torch
    T, H = p.ntok, 96
    log("prefill-backward leg (T=4096)")
    out, lse, _ = m.mla_prefill(dims, q, ckv, ks, w_kv_b, gate, cu, out_dtype=torch.float32, want_lse=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(9)
    dout = torch.randn((T, H * 128), generator=g, dtype=torch.float32, device="cuda")
    need = int(m.lib.mla_prefill_backward_workspace_size(ctypes.byref(dims.c()), T, cu.shape[0] - 1))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    m.mla_prefill_backward(dims, q, ckv, ks, w_kv_b, gate, cu, out, lse, dout, workspace=ws)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        m.mla_prefill_backward(dims, q, ckv, ks, w_kv_b, gate, cu, out, lse, dout, workspace=ws)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    m.mla_timing_enable(True)
    m.mla_prefill_backward(dims, q, ckv, ks, w_kv_b, gate, cu, out, lse, dout, workspace=ws)
    torch.cuda.synchronize()
    kern = {}
    for k in ("bw_plan", "bw_expand", "bw_prep", "bw_dkv", "bw_dq", "bw_dks", "bw_transpose", "bw_weights"):
        tot, n = m.mla_timing_read(k)
        if n:
            kern[k] = tot
    m.mla_timing_enable(False)
    pairs = T * (T + 1) / 2
    # causal pairs: QK^T recompute (192) + dP (128) + dQ (192) + dK (192) + dV (128); expansion recompute,
    # dc^KV and dW (each 2 T H 256 R)
    attn = 2.0 * H * pairs * (192 + 128 + 192 + 192 + 128)
    lat = 3 * 2.0 * T * H * 256 * 512
    # the two attention passes: dK/dV recomputes S and dP (640 MACs per causal pair), dQ recomputes them
    # again (512); matrix-core busy fraction and HBM bytes from the committed counter tables
    passes = {}
    for k, macs in (("bwd_dkv", 640), ("bwd_dq", 512)):
        kms = kern.get("bw_dkv" if k == "bwd_dkv" else "bw_dq")
        if kms:
            tf = 2.0 * H * pairs * macs / (kms * 1e-3) / 1e12
            traffic = recorded_traffic(k, BACKWARD_SOURCES)
            passes[k] = {"ms": round(kms, 4), "tflops": round(tf, 1), "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                         "mfma_busy": recorded_mfma_busy(k, BACKWARD_SOURCES),
                         "traffic_gb": None if traffic is None else round(traffic / 1e9, 3)}
    return {"workload": "backward of the Kimi K3 prefill, B=1 T=4096 H=96 (bf16 operands, fp32 gradients)",
            "ms": round(ms, 4), "gflop_algorithmic": round((attn + lat) / 1e9, 1),
            "tflops": round((attn + lat) / (ms * 1e-3) / 1e12, 2),
            "frac_mfma_peak": round((attn + lat) / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "kernels_ms_per_call": {k: round(v, 4) for k, v in kern.items()}, "passes": passes}


def layer_leg(m, dims, steps: int = 5):
    """The whole gated MLA layer (hidden 7168, q_lora_rank 1536, 96 heads) at
    T = 4096: projections of x, RMSNorms, q up-projection, attention, output
    projection. Seeded random-init weights of that architecture."""
    import torch
    import synth
    L = synth.k3_layer()
    T, hid, qr = L.ntok, L.hidden, L.q_rank
    H, R, S, D, V = 96, 512, 64, 192, 128

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(torch.bfloat16)
    log("whole-layer leg (T=4096, hidden 7168)")
    t = [up(a) for a in (L.x, L.w_dq, L.g_q, L.w_uq, L.w_kv_a, L.g_kv, L.w_kv_b, L.w_g, L.w_o)]
    cu = torch.from_numpy(L.cu_seqlens).cuda()
    out = torch.empty((T, hid), dtype=torch.bfloat16, device="cuda")
    ml = torch.empty(H, dtype=torch.float32, device="cuda")
    ws = torch.empty(m.mla_layer_workspace_size(dims, hid, qr, T, 1), dtype=torch.uint8, device="cuda")

    def call():
        m.mla_layer_forward(dims, *t, cu, out=out, max_logit=ml, workspace=ws)
    for _ in range(2):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        call()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    m.mla_timing_enable(True)
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    kern = {}
    for k in ("layer_proj_x", "layer_norm", "layer_proj_q", "prefill_plan", "prefill_expand", "prefill_attn",
              "prefill_refine_rows", "prefill_refine_score", "layer_proj_o"):
        tot, n = m.mla_timing_read(k)
        if n:
            kern[k] = tot / n
    m.mla_timing_enable(False)
    gf = {"layer_proj_x": 2.0 * T * hid * (qr + R + S + H * V), "layer_proj_q": 2.0 * T * qr * H * D,
          "layer_proj_o": 2.0 * T * H * V * hid}
    qk, pv, ex = prefill_flops(T, H)
    total = sum(gf.values()) + qk + pv + ex
    gx = gf["layer_proj_x"] / (kern["layer_proj_x"] * 1e-3) / 1e12
    return {"workload": "Kimi K3 gated MLA layer, T=4096, hidden 7168, q_lora_rank 1536, H=96, bf16",
            "ms": round(ms, 4), "gflop": round(total / 1e9, 1), "tflops": round(total / (ms * 1e-3) / 1e12, 2),
            "frac_mfma_peak": round(total / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "kernels_ms": {k: round(v, 4) for k, v in kern.items()},
            "roofline": {"kernel": "layer_proj_x", "bound": "mfma", "achieved": round(gx, 2),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(gx / PEAK_BF16_TFLOPS, 4),
                         "traffic": recorded_traffic("layer_proj_x", LAYER_SOURCES),
                         "algorithmic": f"{gf['layer_proj_x'] / 1e9:.1f} GFLOP per launch (x W^T for q_a, kv_a, g)"}}


def clip_stress_leg(m, dims, steps: int = 5):
    """The QK-Clip stress workload (T = 2048, heads 0, 19, 38, 57, 76, 95 with
    their q_b_proj and W_UK blocks x40, tau = 100): the attention pass before
    the clip, the clip itself, and the attention pass after it with the
    queries re-projected through the clipped q_b_proj. The query projection
    q = c^Q W_UQ^T runs on mla_linear and is not timed."""
    import torch
    import synth
    log("QK-Clip stress leg (T=2048, six heads x40)")
    p = synth.k3_clip_stress()
    T, H = p.ntok, dims.heads

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(torch.bfloat16)
    cq, ckv, ks, gate = up(p.cq), up(p.ckv), up(p.ks), up(p.gate)
    wq0, wk0 = up(p.w_q_b), up(p.w_kv_b)
    cu = torch.from_numpy(p.cu_seqlens).cuda()
    out = torch.empty((T, H * 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(m.mla_prefill_workspace_size(dims, m.MLA_BF16, T, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def attention(wq, wk, q_norm=None):
        q = m.mla_linear(cq, wq).view(T, H, 192)
        ml = torch.empty(H, dtype=torch.float32, device="cuda")
        m.mla_prefill(dims, q, ckv, ks, wk, gate, cu, out=out, max_logit=ml, workspace=ws, q_norm=q_norm)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(steps):
            m.mla_prefill(dims, q, ckv, ks, wk, gate, cu, out=out, max_logit=ml, workspace=ws, q_norm=q_norm)
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / steps, ml.cpu().numpy().astype(np.float64)

    before_ms, sm0 = attention(wq0, wk0)
    # the QK-norm variant on the same weights (per-head RMSNorm of the queries, unit weight)
    norm_ms, smn = attention(wq0, wk0, q_norm=(None, 1e-6))
    # the clip, timed on fresh copies of the weights (it rescales them in place)
    clip_ms = []
    wq, wk = wq0.clone(), wk0.clone()
    ml0 = torch.from_numpy(sm0.astype(np.float32)).cuda()
    for _ in range(steps):
        wq.copy_(wq0)
        wk.copy_(wk0)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        clipped, gamma = m.mla_qk_clip(dims, wq, wk, ml0, synth.TAU)
        ev[1].record(stream)
        torch.cuda.synchronize()
        clip_ms.append(ev[0].elapsed_time(ev[1]))
    after_ms, sm1 = attention(wq, wk)
    pairs = T * (T + 1) // 2
    fl = 2.0 * H * pairs * (192 + 128) + 2.0 * T * H * 256 * 512
    heads = [int(h) for h in np.nonzero(clipped.cpu().numpy())[0]]
    res = {"workload": "QK-Clip stress: Kimi K3 gated MLA prefill T=2048 H=96 bf16, heads 0,19,38,57,76,95 "
                       "with q_b_proj and W_UK blocks x40, tau=100",
           "gflop_per_pass": round(fl / 1e9, 1),
           "attn_ms_before_clip": round(before_ms, 4), "attn_ms_after_clip": round(after_ms, 4),
           "tflops_before_clip": round(fl / (before_ms * 1e-3) / 1e12, 2),
           "tflops_after_clip": round(fl / (after_ms * 1e-3) / 1e12, 2),
           "frac_mfma_peak": round(fl / (min(before_ms, after_ms) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "clip_ms": round(float(np.median(clip_ms)), 4),
           "clipped_heads": heads,
           "max_logit_before": {str(h): round(float(sm0[h]), 2) for h in heads},
           "max_logit_after_max": round(float(sm1.max()), 4),
           "max_logit_after_le_tau": bool(np.all(sm1 <= synth.TAU * (1 + 1e-3))),
           "qk_norm": {"attn_ms": round(norm_ms, 4),
                       "max_logit": {str(h): round(float(smn[h]), 2) for h in heads},
                       "heads_above_tau": [int(h) for h in np.nonzero(smn > synth.TAU)[0]]}}
    del cq, ckv, ks, gate, wq0, wk0, wq, wk, out, ws
    torch.cuda.empty_cache()
    return res


def expanded_comparator(m, dims, d, dq, dg, lens, absorbed_ms, absorbed_split_ms, steps: int = 3):
    """The decode workload over a per-head cache (K 192 + V 128 values per head
    and token, the materialised form) instead of the latent rows: the bytes the
    latent cache saves, measured. Same q, gate and lengths; the cache rows are
    seeded N(0,1) draws (the spread of K^C, k^S and V), NaN past each length."""
    import torch
    B, H, cap = d.batch, dims.heads, d.cap
    log(f"expanded-cache comparator: allocating {B * H * cap * 320 * 2 / 1e9:.1f} GB of per-head cache")
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    kc = torch.randn((B, H, cap, 192), generator=g, dtype=torch.bfloat16, device="cuda")
    vc = torch.randn((B, H, cap, 128), generator=g, dtype=torch.bfloat16, device="cuda")
    for b in range(B):
        kc[b, :, int(d.lens[b]):] = float("nan")
        vc[b, :, int(d.lens[b]):] = float("nan")
    out = torch.empty((B, 1, H * 128), dtype=torch.bfloat16, device="cuda")
    ml = torch.empty(H, dtype=torch.float32, device="cuda")
    ws = torch.empty(m.mla_expanded_workspace_size(dims, m.MLA_BF16, B, 1, cap), dtype=torch.uint8, device="cuda")
    m.mla_expanded(dims, dq, kc, vc, lens, dg, out=out, max_logit=ml, workspace=ws)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    m.mla_timing_enable(True)
    t0.record(stream)
    for _ in range(steps):
        m.mla_expanded(dims, dq, kc, vc, lens, dg, out=out, max_logit=ml, workspace=ws)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    split_tot, split_n = m.mla_timing_read("expanded_split")
    comb_tot, comb_n = m.mla_timing_read("expanded_combine")
    m.mla_timing_enable(False)
    cache_bytes = float(d.lens.astype(np.int64).sum()) * H * (192 + 128) * 2
    split_ms = split_tot / max(split_n, 1)
    del kc, vc
    torch.cuda.empty_cache()
    return {"ms": round(ms, 4), "cache_bytes": int(cache_bytes), "cache_gbps": round(cache_bytes / (ms * 1e-3) / 1e9, 1),
            "kernels_ms": {"expanded_split": round(split_ms, 4), "expanded_combine": round(comb_tot / max(comb_n, 1), 4)},
            "roofline": {"kernel": "expanded_split", "bound": "hbm",
                         "achieved": round(cache_bytes / (split_ms * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBPS,
                         "unit": "GB/s", "frac": round(cache_bytes / (split_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                         "traffic": recorded_traffic("expanded_split", EXPANDED_SOURCES)},
            "bytes_vs_latent": round(H * 320 / 576, 2),
            "time_vs_absorbed": round(ms / absorbed_ms, 2) if absorbed_ms else None}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-layer", action="store_true", help="skip the whole-layer leg")
    ap.add_argument("--no-backward", action="store_true", help="skip the prefill-backward leg")
    ap.add_argument("--no-varlen", action="store_true", help="skip the long varlen prefill leg")
    ap.add_argument("--no-clip-stress", action="store_true", help="skip the QK-Clip stress leg (T=2048)")
    ap.add_argument("--no-expanded", action="store_true",
                    help="skip the expanded-cache decode comparator (needs 129 GB of device memory)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="first copy 512 MiB device-to-device once (counter calibration for rocprofv3 --pmc runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the library has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import mla_qk_clip_amd as m
    import synth

    torch.cuda.set_device(0)
    dev = "cuda"

    def up(x, dt=torch.bfloat16):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev).to(dt)

    log("generating the prefill workload (T=4096, H=96)")
    p = synth.k3_prefill()
    dims = m.Dims()
    q, ckv, ks = up(p.q), up(p.ckv), up(p.ks)
    w_kv_b, gate = up(p.w_kv_b), up(p.gate)
    w_q_b = up(synth.k3_q_weight())
    cu = torch.from_numpy(p.cu_seqlens).to(dev)
    T = p.ntok
    out = torch.empty((T, 96 * 128), dtype=torch.float32, device=dev)
    ml = torch.empty(96, dtype=torch.float32, device=dev)
    ws = torch.empty(m.mla_prefill_workspace_size(dims, m.MLA_BF16, T, 1), dtype=torch.uint8, device=dev)
    clipped = torch.empty(96, dtype=torch.uint8, device=dev)
    gamma = torch.empty(96, dtype=torch.float32, device=dev)

    decode = not args.no_decode
    if decode:
        log("generating the decode workload (64 x <=32768 rows x 576)")
        d = synth.k3_decode()
        cache = torch.full((d.batch, d.cap, 576), float("nan"), dtype=torch.bfloat16, device=dev)
        for b in range(d.batch):
            rows = d.cache_rows(b)
            cache[b, :rows.shape[0]] = up(rows)
        dq, dg, dw = up(d.q), up(d.gate), up(d.w_kv_b)
        lens = torch.from_numpy(d.lens).to(dev)
        dout = torch.empty((d.batch, 1, 96 * 128), dtype=torch.bfloat16, device=dev)
        dml = torch.empty(96, dtype=torch.float32, device=dev)
        dws = torch.empty(m.mla_absorbed_workspace_size(dims, m.MLA_BF16, d.batch, 1), dtype=torch.uint8,
                          device=dev)
        cache_bytes = float(d.lens.astype(np.int64).sum()) * 576 * 2

    stream = torch.cuda.current_stream()
    if args.calib_copy:
        # a plain copy of known size: reads and writes 512 MiB each
        src = torch.ones(256 << 20, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        m.mla_prefill(dims, q, ckv, ks, w_kv_b, gate, cu, out=out, max_logit=ml, workspace=ws)
        if ev is not None:
            ev[1].record(stream)
        m.mla_qk_clip(dims, w_q_b, w_kv_b, ml, synth.TAU, clipped=clipped, gamma=gamma)
        if ev is not None:
            ev[2].record(stream)
        if decode:
            m.mla_absorbed(dims, dq, cache, lens, dw, dg, out=dout, max_logit=dml, workspace=dws)
        if ev is not None:
            ev[3].record(stream)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    pre_ms = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
    clip_ms = float(np.median([e[1].elapsed_time(e[2]) for e in evs]))
    dec_ms = float(np.median([e[2].elapsed_time(e[3]) for e in evs])) if decode else None

    # per-kernel averages, measured in a second pass with per-launch events
    log("per-kernel timing pass")
    m.mla_timing_enable(True)
    for _ in range(min(args.steps, 10)):
        step()
    torch.cuda.synchronize()
    kern = {}
    for k in ("fill", "prefill_plan", "prefill_expand", "prefill_attn", "prefill_refine_rows",
              "prefill_refine_score", "qk_clip", "absorb_q", "absorbed_split",
              "absorbed_fixup", "absorbed_finish"):
        tot, n = m.mla_timing_read(k)
        if n:
            kern[k] = tot / n
    m.mla_timing_enable(False)

    qk, pv, ex = prefill_flops(T, 96)
    pre_tflops = (qk + pv + ex) / (pre_ms * 1e-3) / 1e12
    attn_tflops = (qk + pv) / (kern["prefill_attn"] * 1e-3) / 1e12
    res = {
        "metric": METRIC,
        "value": round(pre_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Kimi K3 gated MLA prefill B=1 T=4096 H=96 bf16 (step also runs QK-Clip and "
                               "absorbed decode B=64 cache<=32768x576)",
                   "heads": 96, "kv_rank": 512, "shared": 64, "nope": 128, "v": 128, "seq_len": T},
        "prefill": {"ms": round(pre_ms, 4), "tflops": round(pre_tflops, 2),
                    "frac_mfma_peak": round(pre_tflops / PEAK_BF16_TFLOPS, 4),
                    "gflop": round((qk + pv + ex) / 1e9, 1)},
        "qk_clip": {"ms": round(clip_ms, 4)},
        "kernels_ms": {k: round(v, 4) for k, v in kern.items()},
        "roofline": {"kernel": "prefill_attn", "bound": "mfma", "achieved": round(attn_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic("prefill_attn", PREFILL_SOURCES),
                     "mfma_busy": recorded_mfma_busy("prefill_attn", PREFILL_SOURCES),
                     "algorithmic": f"{(qk + pv) / 1e9:.1f} GFLOP per launch (QK^T + PV)"},
    }
    if decode:
        gbps = cache_bytes / (dec_ms * 1e-3) / 1e9
        split_gbps = cache_bytes / (kern["absorbed_split"] * 1e-3) / 1e9
        res["decode"] = {"ms": round(dec_ms, 4), "cache_gbps": round(gbps, 1),
                         "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4), "cache_bytes": int(cache_bytes),
                         "sum_lens": int(d.lens.sum())}
        res["decode_roofline"] = {"kernel": "absorbed_split", "bound": "hbm", "achieved": round(split_gbps, 1),
                                  "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(split_gbps / PEAK_HBM_GBPS, 4),
                                  "traffic": recorded_traffic("absorbed_split", DECODE_SOURCES),
                                  "mfma_busy": recorded_mfma_busy("absorbed_split", DECODE_SOURCES),
                                  "algorithmic": f"{cache_bytes / 1e9:.4f} GB of cache rows per launch"}
    if not args.no_clip_stress:
        res["clip_stress"] = clip_stress_leg(m, dims)
    if not args.no_layer:
        res["layer"] = layer_leg(m, dims)
    if not args.no_backward:
        res["backward"] = backward_leg(m, dims, p, q, ckv, ks, w_kv_b, gate, cu)
    if not args.no_varlen:
        res["varlen_prefill"] = varlen_leg(m, dims)
    if decode and not args.no_expanded:
        res["expanded_decode"] = expanded_comparator(m, dims, d, dq, dg, lens, dec_ms, kern.get("absorbed_split"))
    if not args.no_cpu_baseline:
        log("CPU oracle baseline")
        res["cpu_baseline"] = cpu_baseline(p)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
