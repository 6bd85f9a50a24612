"""Python binding of libmla (gated no-position MLA, per-head max logit, QK-Clip)
for AMD Instinct MI355X (gfx950).

Argument marshalling only: every step runs in the HIP kernels of
``libmla.so``. PyTorch provides device memory and the current HIP stream.
Names match the C ABI in ``include/mla.h``. The library must have been built
(``python mla_qk_clip_amd/build.py``); importing this package without it raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla.so")

MLA_OK, MLA_ERR_INVALID, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE, MLA_ERR_HIP = range(5)
MLA_F32, MLA_BF16 = 0, 1

EXPORTED = (
    "mla_prefill_workspace_size", "mla_prefill", "mla_absorbed_workspace_size", "mla_absorbed",
    "mla_absorbed_noalloc",
    "mla_expanded_workspace_size", "mla_expanded", "mla_linear", "mla_rms_norm", "mla_layer_workspace_size",
    "mla_layer_forward", "mla_prefill_backward_workspace_size", "mla_prefill_backward", "mla_qk_clip", "mla_status_string", "mla_last_error", "mla_version", "mla_timing_enable",
    "mla_timing_read",
)


class MlaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libmla status {status}: {msg}")
        self.status = status


class mla_dims(ctypes.Structure):
    _fields_ = [("heads", ctypes.c_int32), ("kv_rank", ctypes.c_int32), ("shared_dim", ctypes.c_int32),
                ("nope_dim", ctypes.c_int32), ("v_dim", ctypes.c_int32), ("scale", ctypes.c_float)]


class mla_qk_norm(ctypes.Structure):
    _fields_ = [("weight", ctypes.c_void_p), ("eps", ctypes.c_float)]


@dataclass(frozen=True)
class Dims:
    heads: int = 96
    kv_rank: int = 512
    shared_dim: int = 64
    nope_dim: int = 128
    v_dim: int = 128
    scale: float = 0.0   # 0 -> (nope + shared) ** -0.5

    def c(self) -> mla_dims:
        return mla_dims(self.heads, self.kv_rank, self.shared_dim, self.nope_dim, self.v_dim, self.scale)

    @property
    def qk_dim(self) -> int:
        return self.nope_dim + self.shared_dim


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python mla_qk_clip_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    D = ctypes.POINTER(mla_dims)
    lib.mla_prefill_workspace_size.argtypes = [D, I32, I64, I32]
    lib.mla_prefill_workspace_size.restype = SZ
    QN = ctypes.POINTER(mla_qk_norm)
    lib.mla_prefill.argtypes = [D, I32, I32, P, P, P, P, P, QN, P, I32, I64, P, P, P, I32, P, SZ, P]
    lib.mla_prefill.restype = I32
    lib.mla_absorbed_workspace_size.argtypes = [D, I32, I32, I32]
    lib.mla_absorbed_workspace_size.restype = SZ
    lib.mla_absorbed.argtypes = [D, I32, I32, P, P, I64, P, I32, I32, P, P, QN, P, P, I32, P, SZ, P]
    lib.mla_absorbed.restype = I32
    lib.mla_absorbed_noalloc.argtypes = [D, I32, I32, P, P, I64, P, I32, I32, P, P, QN, P, P, I32, P]
    lib.mla_absorbed_noalloc.restype = I32
    lib.mla_expanded_workspace_size.argtypes = [D, I32, I32, I32, I64]
    lib.mla_expanded_workspace_size.restype = SZ
    lib.mla_expanded.argtypes = [D, I32, I32, P, P, P, I64, P, I32, I32, P, P, P, I32, P, SZ, P]
    lib.mla_expanded.restype = I32
    lib.mla_linear.argtypes = [I32, P, I64, I32, P, I32, P, P]
    lib.mla_linear.restype = I32
    lib.mla_rms_norm.argtypes = [I32, P, I64, I32, P, F, P, P]
    lib.mla_rms_norm.restype = I32
    lib.mla_layer_workspace_size.argtypes = [D, I32, I32, I64, I32]
    lib.mla_layer_workspace_size.restype = SZ
    lib.mla_layer_forward.argtypes = [D, I32, I32, F, P, P, P, P, P, P, P, P, P, P, I32, I64, P, P, I32, P, SZ, P]
    lib.mla_layer_forward.restype = I32
    lib.mla_prefill_backward_workspace_size.argtypes = [D, I64, I32]
    lib.mla_prefill_backward_workspace_size.restype = SZ
    lib.mla_prefill_backward.argtypes = [D, P, P, P, P, P, P, I32, I64, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.mla_prefill_backward.restype = I32
    lib.mla_qk_clip.argtypes = [D, I32, P, I32, P, P, F, P, P, P]
    lib.mla_qk_clip.restype = I32
    lib.mla_status_string.argtypes = [I32]
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_last_error.argtypes = []
    lib.mla_last_error.restype = ctypes.c_char_p
    lib.mla_version.argtypes = []
    lib.mla_version.restype = ctypes.c_char_p
    lib.mla_timing_enable.argtypes = [I32]
    lib.mla_timing_enable.restype = None
    lib.mla_timing_read.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I64)]
    lib.mla_timing_read.restype = I32
    return lib


lib = _load()


def _check(status: int):
    if status != MLA_OK:
        raise MlaError(status, f"{lib.mla_status_string(status).decode()}: {lib.mla_last_error().decode()}")


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MLA_BF16
    if t.dtype == torch.float32:
        return MLA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _expect(name: str, t, shape, dtype, optional: bool = False):
    """The C ABI takes bare pointers and trusts the sizes it is given, so the
    binding checks every tensor against them first: a wrong shape, dtype or
    device raises here instead of letting a kernel read past a buffer."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _qk_norm(q_norm, q, dim: int):
    """(weight [dim] or None, eps) -> a pointer to an mla_qk_norm, or None when the variant is off."""
    if q_norm is None:
        return None
    w, eps = q_norm
    _expect("q_norm weight", w, (dim,), q.dtype, optional=True)
    return ctypes.pointer(mla_qk_norm(_ptr(w), float(eps)))


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _torch_dt(code: int):
    return torch.bfloat16 if code == MLA_BF16 else torch.float32


def mla_prefill_workspace_size(dims: Dims, in_dtype: int, total_tokens: int, nseq: int) -> int:
    return int(lib.mla_prefill_workspace_size(ctypes.byref(dims.c()), in_dtype, total_tokens, nseq))


def mla_absorbed_workspace_size(dims: Dims, in_dtype: int, batch: int, tq: int) -> int:
    return int(lib.mla_absorbed_workspace_size(ctypes.byref(dims.c()), in_dtype, batch, tq))


def mla_prefill(dims: Dims, q, ckv, ks, w_kv_b, gate, cu_seqlens, *, out_dtype=None, out=None, lse=None,
                max_logit=None, accumulate=False, workspace=None, want_lse=False, q_norm=None, stream=None):
    """Training-form gated MLA over packed sequences (see ``mla_prefill`` in include/mla.h).

    q [T, H, N+S], ckv [T, R], ks [T, S], w_kv_b [H*(N+V), R], gate [T, H*V] or None,
    cu_seqlens int32 [nseq+1] on the device; q_norm = (weight [N+S] or None, eps) selects the
    QK-norm variant. Returns (out [T, H*V], lse or None, max_logit [H]).
    """
    in_dt = _dt(q)
    out_dt = MLA_F32 if out_dtype is None else (MLA_BF16 if out_dtype == torch.bfloat16 else MLA_F32)
    if out is not None and out_dtype is None:
        out_dt = _dt(out)
    if q.dim() != 3:
        raise ValueError(f"q must be [T, H, N+S], got shape {tuple(q.shape)}")
    T = q.shape[0]
    H, R, S = dims.heads, dims.kv_rank, dims.shared_dim
    nseq = cu_seqlens.numel() - 1
    dev = q.device
    _expect("q", q, (T, H, dims.qk_dim), q.dtype)
    _expect("ckv", ckv, (T, R), q.dtype)
    _expect("ks", ks, (T, S), q.dtype)
    _expect("w_kv_b", w_kv_b, (H * (dims.nope_dim + dims.v_dim), R), q.dtype)
    _expect("gate", gate, (T, H * dims.v_dim), q.dtype, optional=True)
    _expect("cu_seqlens", cu_seqlens, (nseq + 1,), torch.int32)
    if out is None:
        out = torch.empty((T, dims.heads * dims.v_dim), dtype=_torch_dt(out_dt), device=dev)
    if lse is None and want_lse:
        lse = torch.empty((dims.heads, T), dtype=torch.float32, device=dev)
    if max_logit is None:
        max_logit = torch.empty(dims.heads, dtype=torch.float32, device=dev)
    _expect("out", out, (T, H * dims.v_dim), _torch_dt(out_dt))
    _expect("lse", lse, (H, T), torch.float32, optional=True)
    _expect("max_logit", max_logit, (H,), torch.float32)
    need = mla_prefill_workspace_size(dims, in_dt, T, nseq)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = lib.mla_prefill(ctypes.byref(dims.c()), in_dt, out_dt, _ptr(q), _ptr(ckv), _ptr(ks), _ptr(w_kv_b),
                         _ptr(gate), _qk_norm(q_norm, q, dims.qk_dim), _ptr(cu_seqlens), nseq, T, _ptr(out),
                         _ptr(lse), _ptr(max_logit),
                         1 if accumulate else 0, _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st)
    return out, lse, max_logit


def mla_absorbed(dims: Dims, q, cache, lens, w_kv_b, gate, *, out_dtype=None, out=None, max_logit=None,
                 accumulate=False, workspace=None, q_norm=None, stream=None):
    """Absorbed-form gated MLA over the latent cache (see ``mla_absorbed`` in include/mla.h).

    q [B, Tq, H, N+S], cache [B, cap, R+S], lens int32 [B] on the device, w_kv_b [H*(N+V), R],
    gate [B, Tq, H*V] or None; q_norm = (weight [N+S] or None, eps) selects the QK-norm variant.
    Returns (out [B, Tq, H*V], max_logit [H]).
    """
    in_dt = _dt(q)
    out_dt = in_dt if out_dtype is None else (MLA_BF16 if out_dtype == torch.bfloat16 else MLA_F32)
    if out is not None and out_dtype is None:
        out_dt = _dt(out)
    if q.dim() != 4 or cache.dim() != 3:
        raise ValueError(f"q must be [B, Tq, H, N+S] and cache [B, cap, R+S], got {tuple(q.shape)}, "
                         f"{tuple(cache.shape)}")
    B, Tq = q.shape[0], q.shape[1]
    cap = cache.shape[1]
    H, R = dims.heads, dims.kv_rank
    dev = q.device
    _expect("q", q, (B, Tq, H, dims.qk_dim), q.dtype)
    _expect("cache", cache, (B, cap, R + dims.shared_dim), q.dtype)
    _expect("lens", lens, (B,), torch.int32)
    _expect("w_kv_b", w_kv_b, (H * (dims.nope_dim + dims.v_dim), R), q.dtype)
    _expect("gate", gate, (B, Tq, H * dims.v_dim), q.dtype, optional=True)
    if out is None:
        out = torch.empty((B, Tq, dims.heads * dims.v_dim), dtype=_torch_dt(out_dt), device=dev)
    if max_logit is None:
        max_logit = torch.empty(dims.heads, dtype=torch.float32, device=dev)
    _expect("out", out, (B, Tq, H * dims.v_dim), _torch_dt(out_dt))
    _expect("max_logit", max_logit, (H,), torch.float32)
    need = mla_absorbed_workspace_size(dims, in_dt, B, Tq)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = lib.mla_absorbed(ctypes.byref(dims.c()), in_dt, out_dt, _ptr(q), _ptr(cache), cap, _ptr(lens), B, Tq,
                          _ptr(w_kv_b), _ptr(gate), _qk_norm(q_norm, q, dims.qk_dim), _ptr(out), _ptr(max_logit),
                          1 if accumulate else 0,
                          _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st)
    return out, max_logit


def mla_absorbed_noalloc(dims: Dims, q, cache, lens, w_kv_b, gate, *, out, max_logit, accumulate=False,
                         q_norm=None, stream=None):
    """``mla_absorbed`` with the library's built-in scratch memory (see ``mla_absorbed_noalloc`` in
    include/mla.h): nothing is allocated, so ``out`` and ``max_logit`` must be given.

    q [B, Tq, H, N+S], cache [B, cap, R+S], lens int32 [B] on the device, w_kv_b [H*(N+V), R],
    gate [B, Tq, H*V] or None, out [B, Tq, H*V] (its dtype selects the output dtype), max_logit [H].
    """
    in_dt = _dt(q)
    out_dt = _dt(out)
    if q.dim() != 4 or cache.dim() != 3:
        raise ValueError(f"q must be [B, Tq, H, N+S] and cache [B, cap, R+S], got {tuple(q.shape)}, "
                         f"{tuple(cache.shape)}")
    B, Tq = q.shape[0], q.shape[1]
    cap = cache.shape[1]
    H, R = dims.heads, dims.kv_rank
    _expect("q", q, (B, Tq, H, dims.qk_dim), q.dtype)
    _expect("cache", cache, (B, cap, R + dims.shared_dim), q.dtype)
    _expect("lens", lens, (B,), torch.int32)
    _expect("w_kv_b", w_kv_b, (H * (dims.nope_dim + dims.v_dim), R), q.dtype)
    _expect("gate", gate, (B, Tq, H * dims.v_dim), q.dtype, optional=True)
    _expect("out", out, (B, Tq, H * dims.v_dim), out.dtype)
    _expect("max_logit", max_logit, (H,), torch.float32)
    st = lib.mla_absorbed_noalloc(ctypes.byref(dims.c()), in_dt, out_dt, _ptr(q), _ptr(cache), cap, _ptr(lens), B,
                                  Tq, _ptr(w_kv_b), _ptr(gate), _qk_norm(q_norm, q, dims.qk_dim), _ptr(out),
                                  _ptr(max_logit), 1 if accumulate else 0, _stream(stream))
    _check(st)
    return out, max_logit


def mla_expanded_workspace_size(dims: Dims, in_dtype: int, batch: int, tq: int, cap: int) -> int:
    return int(lib.mla_expanded_workspace_size(ctypes.byref(dims.c()), in_dtype, batch, tq, cap))


def mla_expanded(dims: Dims, q, k_cache, v_cache, lens, gate, *, out_dtype=None, out=None, max_logit=None,
                 accumulate=False, workspace=None, stream=None):
    """Gated MLA decode over a per-head (expanded) K/V cache (see ``mla_expanded`` in include/mla.h).

    q [B, Tq, H, N+S], k_cache [B, H, cap, N+S], v_cache [B, H, cap, V], lens int32 [B] on the
    device, gate [B, Tq, H*V] or None, all bf16. Returns (out [B, Tq, H*V], max_logit [H]).
    """
    in_dt = _dt(q)
    out_dt = in_dt if out_dtype is None else (MLA_BF16 if out_dtype == torch.bfloat16 else MLA_F32)
    if out is not None and out_dtype is None:
        out_dt = _dt(out)
    if q.dim() != 4 or k_cache.dim() != 4:
        raise ValueError(f"q must be [B, Tq, H, N+S] and k_cache [B, H, cap, N+S], got {tuple(q.shape)}, "
                         f"{tuple(k_cache.shape)}")
    B, Tq = q.shape[0], q.shape[1]
    H, V = dims.heads, dims.v_dim
    cap = k_cache.shape[2]
    dev = q.device
    _expect("q", q, (B, Tq, H, dims.qk_dim), q.dtype)
    _expect("k_cache", k_cache, (B, H, cap, dims.qk_dim), q.dtype)
    _expect("v_cache", v_cache, (B, H, cap, V), q.dtype)
    _expect("lens", lens, (B,), torch.int32)
    _expect("gate", gate, (B, Tq, H * V), q.dtype, optional=True)
    if out is None:
        out = torch.empty((B, Tq, H * V), dtype=_torch_dt(out_dt), device=dev)
    if max_logit is None:
        max_logit = torch.empty(H, dtype=torch.float32, device=dev)
    _expect("out", out, (B, Tq, H * V), _torch_dt(out_dt))
    _expect("max_logit", max_logit, (H,), torch.float32)
    need = mla_expanded_workspace_size(dims, in_dt, B, Tq, cap)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = lib.mla_expanded(ctypes.byref(dims.c()), in_dt, out_dt, _ptr(q), _ptr(k_cache), _ptr(v_cache), cap,
                          _ptr(lens), B, Tq, _ptr(gate), _ptr(out), _ptr(max_logit), 1 if accumulate else 0,
                          _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st)
    return out, max_logit


def mla_linear(x, w, *, out=None, stream=None):
    """y = x W^T (nn.Linear without bias; see ``mla_linear`` in include/mla.h). x [m, k], w [n, k], bf16."""
    if x.dim() != 2 or w.dim() != 2:
        raise ValueError(f"x must be [m, k] and w [n, k], got {tuple(x.shape)}, {tuple(w.shape)}")
    m, k = x.shape
    n = w.shape[0]
    _expect("x", x, (m, k), torch.bfloat16)
    _expect("w", w, (n, k), torch.bfloat16)
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    _expect("out", out, (m, n), torch.bfloat16)
    _check(lib.mla_linear(MLA_BF16, _ptr(x), m, k, _ptr(w), n, _ptr(out), _stream(stream)))
    return out


def mla_rms_norm(x, weight, eps: float, *, out=None, stream=None):
    """RMSNorm over the rows of x [rows, n] with weight [n] (see ``mla_rms_norm`` in include/mla.h), bf16."""
    if x.dim() != 2:
        raise ValueError(f"x must be [rows, n], got {tuple(x.shape)}")
    rows, n = x.shape
    _expect("x", x, (rows, n), torch.bfloat16)
    _expect("weight", weight, (n,), torch.bfloat16)
    if out is None:
        out = torch.empty_like(x)
    _expect("out", out, (rows, n), torch.bfloat16)
    _check(lib.mla_rms_norm(MLA_BF16, _ptr(x), rows, n, _ptr(weight), float(eps), _ptr(out), _stream(stream)))
    return out


def mla_layer_workspace_size(dims: Dims, hidden: int, q_rank: int, total_tokens: int, nseq: int) -> int:
    return int(lib.mla_layer_workspace_size(ctypes.byref(dims.c()), hidden, q_rank, total_tokens, nseq))


def mla_layer_forward(dims: Dims, x, w_dq, g_q, w_uq, w_kv_a, g_kv, w_kv_b, w_g, w_o, cu_seqlens, *, eps=1e-6,
                      out=None, max_logit=None, accumulate=False, workspace=None, stream=None):
    """Delta_attn of the whole gated MLA layer (see ``mla_layer_forward`` in include/mla.h), bf16.

    x [T, hidden]; weights in the nn.Linear layout [out, in]; cu_seqlens int32 [nseq+1] on the device.
    Returns (out [T, hidden], max_logit [H]).
    """
    if x.dim() != 2:
        raise ValueError(f"x must be [tokens, hidden], got {tuple(x.shape)}")
    T, hidden = x.shape
    q_rank = w_dq.shape[0]
    H, R, S, N, V = dims.heads, dims.kv_rank, dims.shared_dim, dims.nope_dim, dims.v_dim
    bf = torch.bfloat16
    _expect("x", x, (T, hidden), bf)
    _expect("w_dq", w_dq, (q_rank, hidden), bf)
    _expect("g_q", g_q, (q_rank,), bf)
    _expect("w_uq", w_uq, (H * (N + S), q_rank), bf)
    _expect("w_kv_a", w_kv_a, (R + S, hidden), bf)
    _expect("g_kv", g_kv, (R,), bf)
    _expect("w_kv_b", w_kv_b, (H * (N + V), R), bf)
    _expect("w_g", w_g, (H * V, hidden), bf)
    _expect("w_o", w_o, (hidden, H * V), bf)
    nseq = cu_seqlens.shape[0] - 1
    _expect("cu_seqlens", cu_seqlens, (nseq + 1,), torch.int32)
    if out is None:
        out = torch.empty((T, hidden), dtype=bf, device=x.device)
    if max_logit is None:
        max_logit = torch.empty(H, dtype=torch.float32, device=x.device)
    _expect("out", out, (T, hidden), bf)
    _expect("max_logit", max_logit, (H,), torch.float32)
    need = mla_layer_workspace_size(dims, hidden, q_rank, T, nseq)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    st = lib.mla_layer_forward(ctypes.byref(dims.c()), hidden, q_rank, float(eps), _ptr(x), _ptr(w_dq), _ptr(g_q),
                               _ptr(w_uq), _ptr(w_kv_a), _ptr(g_kv), _ptr(w_kv_b), _ptr(w_g), _ptr(w_o),
                               _ptr(cu_seqlens), nseq, T, _ptr(out), _ptr(max_logit), 1 if accumulate else 0,
                               _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st)
    return out, max_logit


def mla_prefill_backward(dims: Dims, q, ckv, ks, w_kv_b, gate, cu_seqlens, out, lse, dout, *, workspace=None,
                         stream=None):
    """Gradients of the training-form prefill (see ``mla_prefill_backward`` in include/mla.h).

    q [T, H, N+S], ckv [T, R], ks [T, S], w_kv_b [H*(N+V), R], gate [T, H*V] or None (bf16); cu_seqlens
    int32 [nseq+1] on the device; out [T, H*V] and lse [H, T] from the forward (fp32); dout [T, H*V] fp32.
    Returns (dq, dckv, dks, dw_kv_b, dgate or None), fp32 device tensors. Nothing is read back to the host.
    """
    T = q.shape[0]
    H, R, S, N, V = dims.heads, dims.kv_rank, dims.shared_dim, dims.nope_dim, dims.v_dim
    bf, f32 = torch.bfloat16, torch.float32
    _expect("q", q, (T, H, N + S), bf)
    _expect("ckv", ckv, (T, R), bf)
    _expect("ks", ks, (T, S), bf)
    _expect("w_kv_b", w_kv_b, (H * (N + V), R), bf)
    _expect("gate", gate, (T, H * V), bf, optional=True)
    _expect("out", out, (T, H * V), f32)
    _expect("lse", lse, (H, T), f32)
    _expect("dout", dout, (T, H * V), f32)
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_cuda:
        raise ValueError("cu_seqlens must be a 1-D int32 device tensor")
    nseq = cu_seqlens.shape[0] - 1
    dev = q.device
    dq = torch.empty((T, H, N + S), dtype=f32, device=dev)
    dckv = torch.empty((T, R), dtype=f32, device=dev)
    dks = torch.empty((T, S), dtype=f32, device=dev)
    dw = torch.empty((H * (N + V), R), dtype=f32, device=dev)
    dg = torch.empty((T, H * V), dtype=f32, device=dev) if gate is not None else None
    need = int(lib.mla_prefill_backward_workspace_size(ctypes.byref(dims.c()), T, nseq))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = lib.mla_prefill_backward(ctypes.byref(dims.c()), _ptr(q), _ptr(ckv), _ptr(ks), _ptr(w_kv_b), _ptr(gate),
                                  _ptr(cu_seqlens), nseq, T, _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dckv),
                                  _ptr(dks), _ptr(dw), _ptr(dg), _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st)
    return dq, dckv, dks, dw, dg


def mla_qk_clip(dims: Dims, w_q_b, w_kv_b, max_logit, tau: float, *, clipped=None, gamma=None, stream=None):
    """QK-Clip in place on q_b_proj.weight [H*D, q_in] and kv_b_proj.weight [H*(N+V), R].

    Returns (clipped uint8 [H], gamma fp32 [H]).
    """
    dev = w_q_b.device
    H = dims.heads
    if w_q_b.dim() != 2:
        raise ValueError(f"w_q_b must be [H*(N+S), q_in], got shape {tuple(w_q_b.shape)}")
    _expect("w_q_b", w_q_b, (H * dims.qk_dim, w_q_b.shape[1]), w_q_b.dtype)
    _expect("w_kv_b", w_kv_b, (H * (dims.nope_dim + dims.v_dim), dims.kv_rank), w_q_b.dtype)
    _expect("max_logit", max_logit, (H,), torch.float32)
    if clipped is None:
        clipped = torch.empty(H, dtype=torch.uint8, device=dev)
    if gamma is None:
        gamma = torch.empty(H, dtype=torch.float32, device=dev)
    _expect("clipped", clipped, (H,), torch.uint8)
    _expect("gamma", gamma, (H,), torch.float32)
    st = lib.mla_qk_clip(ctypes.byref(dims.c()), _dt(w_q_b), _ptr(w_q_b), w_q_b.shape[1], _ptr(w_kv_b),
                         _ptr(max_logit), float(tau), _ptr(clipped), _ptr(gamma), _stream(stream))
    _check(st)
    return clipped, gamma


def mla_timing_enable(on: bool) -> None:
    lib.mla_timing_enable(1 if on else 0)


def mla_timing_read(kernel: str):
    """(total milliseconds, launches) of one kernel since timing was enabled."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    lib.mla_timing_read(kernel.encode(), ctypes.byref(ms), ctypes.byref(n))
    return ms.value, n.value
