// C ABI front end of libmla: argument validation, workspace sizing and
// dispatch to the gfx950 kernels. Nothing is launched before every argument
// has been checked; no exception leaves this file.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "mla.h"
#include "mla_internal.h"

namespace {

thread_local std::string g_last_error;

mla_status fail(mla_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
mla_status fail(mla_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

mla_status hip_fail(hipError_t e, const char* where) {
  return fail(MLA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Shape {
  int H, R, S, N, V;
  float scale;
};

mla_status check_dims(const mla_dims* d, mla_dtype in, Shape* out) {
  if (!d) return fail(MLA_ERR_INVALID, "dims is NULL");
  if (d->heads < 1 || d->kv_rank < 1 || d->shared_dim < 0 || d->nope_dim < 1 || d->v_dim < 1)
    return fail(MLA_ERR_INVALID, "dims must be positive (heads=%d kv_rank=%d shared=%d nope=%d v=%d)", d->heads,
                d->kv_rank, d->shared_dim, d->nope_dim, d->v_dim);
  if (!(d->scale >= 0.0f) || !isfinite(d->scale)) return fail(MLA_ERR_INVALID, "scale must be finite and >= 0");
  if (in == MLA_BF16) {
    if (d->kv_rank != mla::kR || d->shared_dim != mla::kS || d->nope_dim != mla::kN || d->v_dim != mla::kV)
      return fail(MLA_ERR_UNSUPPORTED,
                  "bf16 kernels are compiled for kv_rank=512 shared=64 nope=128 v=128 (got %d %d %d %d)",
                  d->kv_rank, d->shared_dim, d->nope_dim, d->v_dim);
  } else if (in == MLA_F32) {
    if (d->kv_rank > 1024 || d->nope_dim + d->shared_dim > 256 || d->v_dim > 256)
      return fail(MLA_ERR_UNSUPPORTED, "fp32 kernels need kv_rank <= 1024, nope + shared <= 256, v <= 256");
  } else {
    return fail(MLA_ERR_INVALID, "unknown dtype %d", static_cast<int>(in));
  }
  out->H = d->heads;
  out->R = d->kv_rank;
  out->S = d->shared_dim;
  out->N = d->nope_dim;
  out->V = d->v_dim;
  out->scale = d->scale > 0.0f ? d->scale : 1.0f / sqrtf(static_cast<float>(d->nope_dim + d->shared_dim));
  return MLA_OK;
}

#define REQUIRE_PTR(p, align)                                                              \
  do {                                                                                     \
    if (!(p)) return fail(MLA_ERR_INVALID, "%s is NULL", #p);                              \
    if (!aligned((p), (align))) return fail(MLA_ERR_INVALID, "%s is not %d-byte aligned", #p, (align)); \
  } while (0)
#define OPTIONAL_PTR(p, align)                                                             \
  do {                                                                                     \
    if ((p) && !aligned((p), (align))) return fail(MLA_ERR_INVALID, "%s is not %d-byte aligned", #p, (align)); \
  } while (0)

// The optional QK-norm argument: eps finite and >= 0, the weight (if any) aligned.
mla_status check_qk_norm(const mla_qk_norm* qn, mla::QNorm* out) {
  *out = mla::QNorm{};
  if (!qn) return MLA_OK;
  if (!(qn->eps >= 0.0f) || !isfinite(qn->eps)) return fail(MLA_ERR_INVALID, "q_norm eps must be finite and >= 0");
  if (qn->weight && !aligned(qn->weight, 16)) return fail(MLA_ERR_INVALID, "q_norm weight is not 16-byte aligned");
  out->w = qn->weight;
  out->eps = qn->eps;
  out->on = true;
  return MLA_OK;
}

// Checks of an absorbed-form call other than its workspace (shared by the
// caller-workspace and the built-in-scratch entry points).
mla_status check_absorbed(const mla_dims* dims, mla_dtype in_dtype, mla_dtype out_dtype, const void* q,
                          const void* cache, int64_t cap, const int32_t* lens, int32_t batch, int32_t tq,
                          const void* w_kv_b, const void* gate, const mla_qk_norm* q_norm, void* out,
                          float* max_logit, int32_t accumulate, Shape* s, mla::QNorm* qn) {
  mla_status st = check_dims(dims, in_dtype, s);
  if (st != MLA_OK) return st;
  st = check_qk_norm(q_norm, qn);
  if (st != MLA_OK) return st;
  if (out_dtype != MLA_F32 && out_dtype != MLA_BF16) return fail(MLA_ERR_INVALID, "unknown out_dtype");
  if (in_dtype == MLA_F32 && out_dtype != MLA_F32)
    return fail(MLA_ERR_UNSUPPORTED, "fp32 inputs produce fp32 outputs only");
  if (batch < 0 || tq < 1) return fail(MLA_ERR_INVALID, "batch must be >= 0 and tq >= 1");
  if (cap < tq) return fail(MLA_ERR_INVALID, "cap (%lld) must be >= tq (%d)", static_cast<long long>(cap), tq);
  if (cap > INT32_MAX) return fail(MLA_ERR_UNSUPPORTED, "cap above 2^31 - 1");
  if (accumulate != 0 && accumulate != 1) return fail(MLA_ERR_INVALID, "accumulate must be 0 or 1");
  if (in_dtype == MLA_BF16 && s->H > mla::kDecMaxHeads)
    return fail(MLA_ERR_UNSUPPORTED, "bf16 absorbed kernel supports up to %d heads", mla::kDecMaxHeads);
  if (static_cast<int64_t>(batch) * tq > (int64_t{1} << 24)) return fail(MLA_ERR_UNSUPPORTED, "batch * tq above 2^24");
  REQUIRE_PTR(max_logit, 4);
  if (batch > 0) {
    REQUIRE_PTR(q, 16);
    REQUIRE_PTR(cache, 16);
    REQUIRE_PTR(lens, 4);
    REQUIRE_PTR(w_kv_b, 16);
    REQUIRE_PTR(out, 16);
    OPTIONAL_PTR(gate, 16);
  }
  return MLA_OK;
}

mla_status run_absorbed(const Shape& s, mla_dtype in_dtype, mla_dtype out_dtype, const void* q, const void* cache,
                        int64_t cap, const int32_t* lens, int32_t batch, int32_t tq, const void* w_kv_b,
                        const void* gate, const mla::QNorm& qn, void* out, float* max_logit, int32_t accumulate,
                        void* workspace, hipStream_t stream) {
  hipError_t e = hipSuccess;
  // the bf16 path clears the max-logit slots in its first kernel
  const bool fused_init = in_dtype == MLA_BF16 && batch > 0;
  if (!accumulate && !fused_init) {
    e = mla::launch_fill(max_logit, s.H, -INFINITY, stream);
    if (e != hipSuccess) return hip_fail(e, "max_logit init");
  }
  if (batch == 0) return MLA_OK;
  if (in_dtype == MLA_BF16) {
    e = mla::launch_absorbed_bf16(s.H, s.scale, out_dtype == MLA_BF16, q, cache, cap, lens, batch, tq, w_kv_b,
                                  gate, out, max_logit, !accumulate, workspace, stream, qn);
  } else {
    e = mla::launch_absorbed_f32(s.H, s.R, s.S, s.N, s.V, s.scale, static_cast<const float*>(q),
                                 static_cast<const float*>(cache), cap, lens, batch, tq,
                                 static_cast<const float*>(w_kv_b), static_cast<const float*>(gate),
                                 static_cast<float*>(out), max_logit, stream, qn);
  }
  if (e != hipSuccess) return hip_fail(e, "mla_absorbed launch");
  return MLA_OK;
}

// Scratch memory of mla_absorbed_noalloc: one static device array, which every
// GPU the library runs on holds (its own copy, at its own address) until the
// process ends. In host code `scratch` names a host-side stand-in, not device
// memory: its device address is looked up once per device with
// hipGetSymbolAddress (that device current) and only that address is used.
constexpr size_t kScratchBytes = size_t{128} << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

hipError_t scratch_of_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MLA_ERR_WORKSPACE: return "workspace too small";
    case MLA_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* mla_last_error(void) { return g_last_error.c_str(); }

const char* mla_version(void) { return "libmla 0.1 (gfx950)"; }

size_t mla_prefill_workspace_size(const mla_dims* dims, mla_dtype in_dtype, int64_t total_tokens, int32_t nseq) {
  Shape s;
  if (check_dims(dims, in_dtype, &s) != MLA_OK || total_tokens < 0 || nseq < 0) return 0;
  if (in_dtype == MLA_BF16) return mla::prefill_ws_layout(s.H, total_tokens, nseq).total;
  return mla::prefill_f32_ws(s.H, total_tokens, s.N, s.V);
}

mla_status mla_prefill(const mla_dims* dims, mla_dtype in_dtype, mla_dtype out_dtype, const void* q,
                       const void* ckv, const void* ks, const void* w_kv_b, const void* gate,
                       const mla_qk_norm* q_norm, const int32_t* cu_seqlens, int32_t nseq, int64_t total_tokens,
                       void* out, float* lse, float* max_logit, int32_t accumulate, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  g_last_error.clear();
  Shape s;
  mla_status st = check_dims(dims, in_dtype, &s);
  if (st != MLA_OK) return st;
  mla::QNorm qn;
  st = check_qk_norm(q_norm, &qn);
  if (st != MLA_OK) return st;
  if (out_dtype != MLA_F32 && out_dtype != MLA_BF16) return fail(MLA_ERR_INVALID, "unknown out_dtype");
  if (in_dtype == MLA_F32 && out_dtype != MLA_F32)
    return fail(MLA_ERR_UNSUPPORTED, "fp32 inputs produce fp32 outputs only");
  if (nseq < 0 || total_tokens < 0) return fail(MLA_ERR_INVALID, "nseq and total_tokens must be >= 0");
  if (nseq == 0 && total_tokens != 0) return fail(MLA_ERR_INVALID, "total_tokens > 0 needs nseq >= 1");
  if (total_tokens > (int64_t{1} << 30)) return fail(MLA_ERR_UNSUPPORTED, "total_tokens above 2^30");
  if (accumulate != 0 && accumulate != 1) return fail(MLA_ERR_INVALID, "accumulate must be 0 or 1");
  REQUIRE_PTR(max_logit, 4);
  OPTIONAL_PTR(lse, 4);
  if (total_tokens > 0) {
    REQUIRE_PTR(q, 16);
    REQUIRE_PTR(ckv, 16);
    REQUIRE_PTR(ks, 16);
    REQUIRE_PTR(w_kv_b, 16);
    REQUIRE_PTR(out, 16);
    REQUIRE_PTR(cu_seqlens, 4);
    OPTIONAL_PTR(gate, 16);
    const size_t need = mla_prefill_workspace_size(dims, in_dtype, total_tokens, nseq);
    if (!workspace || workspace_bytes < need)
      return fail(MLA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                  workspace ? workspace_bytes : static_cast<size_t>(0));
    if (!aligned(workspace, 16)) return fail(MLA_ERR_INVALID, "workspace is not 16-byte aligned");
  }

  hipError_t e = hipSuccess;
  // the bf16 path clears the max-logit slots in its first kernel
  const bool fused_init = in_dtype == MLA_BF16 && total_tokens > 0;
  if (!accumulate && !fused_init) {
    e = mla::launch_fill(max_logit, s.H, -INFINITY, stream);
    if (e != hipSuccess) return hip_fail(e, "max_logit init");
  }
  if (total_tokens == 0) return MLA_OK;
  if (in_dtype == MLA_BF16) {
    e = mla::launch_prefill_bf16(s.H, s.scale, out_dtype == MLA_BF16, q, ckv, ks, w_kv_b, gate, cu_seqlens, nseq,
                                 total_tokens, out, lse, max_logit, !accumulate, workspace, stream, qn);
  } else {
    e = mla::launch_prefill_f32(s.H, s.R, s.S, s.N, s.V, s.scale, static_cast<const float*>(q),
                                static_cast<const float*>(ckv), static_cast<const float*>(ks),
                                static_cast<const float*>(w_kv_b), static_cast<const float*>(gate), cu_seqlens,
                                nseq, total_tokens, static_cast<float*>(out), lse, max_logit, workspace, stream,
                                qn);
  }
  if (e != hipSuccess) return hip_fail(e, "mla_prefill launch");
  return MLA_OK;
}

size_t mla_absorbed_workspace_size(const mla_dims* dims, mla_dtype in_dtype, int32_t batch, int32_t tq) {
  Shape s;
  if (check_dims(dims, in_dtype, &s) != MLA_OK || batch < 0 || tq < 0) return 0;
  if (in_dtype == MLA_BF16) return mla::absorbed_ws_layout(s.H, batch, tq).total;
  return 0;
}

mla_status mla_absorbed(const mla_dims* dims, mla_dtype in_dtype, mla_dtype out_dtype, const void* q,
                        const void* cache, int64_t cap, const int32_t* lens, int32_t batch, int32_t tq,
                        const void* w_kv_b, const void* gate, const mla_qk_norm* q_norm, void* out,
                        float* max_logit, int32_t accumulate, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  g_last_error.clear();
  Shape s;
  mla::QNorm qn;
  mla_status st = check_absorbed(dims, in_dtype, out_dtype, q, cache, cap, lens, batch, tq, w_kv_b, gate, q_norm,
                                 out, max_logit, accumulate, &s, &qn);
  if (st != MLA_OK) return st;
  if (batch > 0) {
    const size_t need = mla_absorbed_workspace_size(dims, in_dtype, batch, tq);
    if (need > 0) {
      if (!workspace || workspace_bytes < need)
        return fail(MLA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : static_cast<size_t>(0));
      if (!aligned(workspace, 16)) return fail(MLA_ERR_INVALID, "workspace is not 16-byte aligned");
    }
  }
  return run_absorbed(s, in_dtype, out_dtype, q, cache, cap, lens, batch, tq, w_kv_b, gate, qn, out, max_logit,
                      accumulate, workspace, stream);
}

mla_status mla_absorbed_noalloc(const mla_dims* dims, mla_dtype in_dtype, mla_dtype out_dtype, const void* q,
                                const void* cache, int64_t cap, const int32_t* lens, int32_t batch, int32_t tq,
                                const void* w_kv_b, const void* gate, const mla_qk_norm* q_norm, void* out,
                                float* max_logit, int32_t accumulate, hipStream_t stream) {
  g_last_error.clear();
  Shape s;
  mla::QNorm qn;
  mla_status st = check_absorbed(dims, in_dtype, out_dtype, q, cache, cap, lens, batch, tq, w_kv_b, gate, q_norm,
                                 out, max_logit, accumulate, &s, &qn);
  if (st != MLA_OK) return st;
  const size_t need = batch > 0 ? mla_absorbed_workspace_size(dims, in_dtype, batch, tq) : 0;
  if (need > kScratchBytes)
    return fail(MLA_ERR_UNSUPPORTED,
                "mla_absorbed_noalloc: these sizes need %zu bytes of scratch, the built-in scratch holds %zu "
                "(use mla_absorbed with a caller workspace)",
                need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = scratch_of_current_device(&ws);
    if (e != hipSuccess) return hip_fail(e, "mla_absorbed_noalloc: scratch address");
  }
  return run_absorbed(s, in_dtype, out_dtype, q, cache, cap, lens, batch, tq, w_kv_b, gate, qn, out, max_logit,
                      accumulate, ws, stream);
}

size_t mla_expanded_workspace_size(const mla_dims* dims, mla_dtype in_dtype, int32_t batch, int32_t tq,
                                   int64_t cap) {
  Shape s;
  if (in_dtype != MLA_BF16 || check_dims(dims, in_dtype, &s) != MLA_OK || batch < 0 || tq < 0 || cap < 0 ||
      cap > (int64_t{1} << 27))
    return 0;
  return mla::expanded_ws_layout(s.H, batch, tq, cap).total;
}

mla_status mla_expanded(const mla_dims* dims, mla_dtype in_dtype, mla_dtype out_dtype, const void* q,
                        const void* k_cache, const void* v_cache, int64_t cap, const int32_t* lens, int32_t batch,
                        int32_t tq, const void* gate, void* out, float* max_logit, int32_t accumulate,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_last_error.clear();
  if (in_dtype != MLA_BF16) return fail(MLA_ERR_UNSUPPORTED, "the expanded-cache decode takes bf16 inputs only");
  Shape s;
  mla_status st = check_dims(dims, in_dtype, &s);
  if (st != MLA_OK) return st;
  if (out_dtype != MLA_F32 && out_dtype != MLA_BF16) return fail(MLA_ERR_INVALID, "unknown out_dtype");
  if (batch < 0 || tq < 1) return fail(MLA_ERR_INVALID, "batch must be >= 0 and tq >= 1");
  if (cap < tq) return fail(MLA_ERR_INVALID, "cap (%lld) must be >= tq (%d)", static_cast<long long>(cap), tq);
  if (cap > (int64_t{1} << 27)) return fail(MLA_ERR_UNSUPPORTED, "cap above 2^27");
  if (accumulate != 0 && accumulate != 1) return fail(MLA_ERR_INVALID, "accumulate must be 0 or 1");
  if (static_cast<int64_t>(batch) * tq * ((s.H + 3) / 4) > INT32_MAX)
    return fail(MLA_ERR_UNSUPPORTED, "batch * tq * heads too large");
  REQUIRE_PTR(max_logit, 4);
  if (batch > 0) {
    REQUIRE_PTR(q, 16);
    REQUIRE_PTR(k_cache, 16);
    REQUIRE_PTR(v_cache, 16);
    REQUIRE_PTR(lens, 4);
    REQUIRE_PTR(out, 16);
    OPTIONAL_PTR(gate, 16);
    const size_t need = mla_expanded_workspace_size(dims, in_dtype, batch, tq, cap);
    if (!workspace || workspace_bytes < need)
      return fail(MLA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                  workspace ? workspace_bytes : static_cast<size_t>(0));
    if (!aligned(workspace, 16)) return fail(MLA_ERR_INVALID, "workspace is not 16-byte aligned");
  }
  hipError_t e = hipSuccess;
  if (!accumulate) {
    e = mla::launch_fill(max_logit, s.H, -INFINITY, stream);
    if (e != hipSuccess) return hip_fail(e, "max_logit init");
  }
  if (batch == 0) return MLA_OK;
  e = mla::launch_expanded_bf16(s.H, s.scale, out_dtype == MLA_BF16, q, k_cache, v_cache, cap, lens, batch, tq, gate,
                                out, max_logit, workspace, stream);
  if (e != hipSuccess) return hip_fail(e, "mla_expanded launch");
  return MLA_OK;
}

mla_status mla_linear(mla_dtype dtype, const void* x, int64_t m, int32_t k, const void* w, int32_t n, void* y,
                      hipStream_t stream) {
  g_last_error.clear();
  if (dtype != MLA_BF16) return fail(MLA_ERR_UNSUPPORTED, "mla_linear takes bf16 only");
  if (m < 0 || m > (int64_t{1} << 30)) return fail(MLA_ERR_INVALID, "m must be in [0, 2^30]");
  if (k < 128 || k % 128 != 0 || k > 65536)
    return fail(MLA_ERR_UNSUPPORTED, "k must be a multiple of 128 in [128, 65536]");
  if (n < 8 || n % 8 != 0) return fail(MLA_ERR_UNSUPPORTED, "n must be a positive multiple of 8");
  if (m == 0) return MLA_OK;
  REQUIRE_PTR(x, 16);
  REQUIRE_PTR(w, 16);
  REQUIRE_PTR(y, 16);
  const hipError_t e = mla::launch_linear_bf16(x, m, k, w, n, y, stream);
  if (e != hipSuccess) return hip_fail(e, "mla_linear launch");
  return MLA_OK;
}

mla_status mla_rms_norm(mla_dtype dtype, const void* x, int64_t rows, int32_t n, const void* weight, float eps,
                        void* y, hipStream_t stream) {
  g_last_error.clear();
  if (dtype != MLA_BF16) return fail(MLA_ERR_UNSUPPORTED, "mla_rms_norm takes bf16 only");
  if (rows < 0) return fail(MLA_ERR_INVALID, "rows must be >= 0");
  if (n < 8 || n % 8 != 0 || n > 2048) return fail(MLA_ERR_UNSUPPORTED, "n must be a multiple of 8 in [8, 2048]");
  if (!(eps >= 0.0f) || !isfinite(eps)) return fail(MLA_ERR_INVALID, "eps must be finite and >= 0");
  if (rows == 0) return MLA_OK;
  REQUIRE_PTR(x, 16);
  REQUIRE_PTR(weight, 16);
  REQUIRE_PTR(y, 16);
  const hipError_t e = mla::launch_rms_norm_bf16(x, rows, n, weight, eps, y, stream);
  if (e != hipSuccess) return hip_fail(e, "mla_rms_norm launch");
  return MLA_OK;
}

size_t mla_layer_workspace_size(const mla_dims* dims, int32_t hidden, int32_t q_rank, int64_t total_tokens,
                                int32_t nseq) {
  Shape s;
  if (check_dims(dims, MLA_BF16, &s) != MLA_OK || hidden < 128 || q_rank < 128 || total_tokens < 0 || nseq < 0)
    return 0;
  return mla::layer_ws_layout(s.H, hidden, q_rank, total_tokens, nseq).total;
}

mla_status mla_layer_forward(const mla_dims* dims, int32_t hidden, int32_t q_rank, float eps, const void* x,
                             const void* w_dq, const void* g_q, const void* w_uq, const void* w_kv_a,
                             const void* g_kv, const void* w_kv_b, const void* w_g, const void* w_o,
                             const int32_t* cu_seqlens, int32_t nseq, int64_t total_tokens, void* out,
                             float* max_logit, int32_t accumulate, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  g_last_error.clear();
  Shape s;
  mla_status st = check_dims(dims, MLA_BF16, &s);
  if (st != MLA_OK) return st;
  if (hidden < 128 || hidden % 128 != 0 || hidden > 65536)
    return fail(MLA_ERR_UNSUPPORTED, "hidden must be a multiple of 128 in [128, 65536]");
  if (q_rank < 128 || q_rank % 128 != 0 || q_rank > 2048)
    return fail(MLA_ERR_UNSUPPORTED, "q_rank must be a multiple of 128 in [128, 2048]");
  if (!(eps >= 0.0f) || !isfinite(eps)) return fail(MLA_ERR_INVALID, "eps must be finite and >= 0");
  if (nseq < 0 || total_tokens < 0) return fail(MLA_ERR_INVALID, "nseq and total_tokens must be >= 0");
  if (nseq == 0 && total_tokens != 0) return fail(MLA_ERR_INVALID, "total_tokens > 0 needs nseq >= 1");
  if (total_tokens > (int64_t{1} << 30)) return fail(MLA_ERR_UNSUPPORTED, "total_tokens above 2^30");
  if (accumulate != 0 && accumulate != 1) return fail(MLA_ERR_INVALID, "accumulate must be 0 or 1");
  REQUIRE_PTR(max_logit, 4);
  if (total_tokens > 0) {
    REQUIRE_PTR(x, 16);
    REQUIRE_PTR(w_dq, 16);
    REQUIRE_PTR(g_q, 16);
    REQUIRE_PTR(w_uq, 16);
    REQUIRE_PTR(w_kv_a, 16);
    REQUIRE_PTR(g_kv, 16);
    REQUIRE_PTR(w_kv_b, 16);
    REQUIRE_PTR(w_g, 16);
    REQUIRE_PTR(w_o, 16);
    REQUIRE_PTR(cu_seqlens, 4);
    REQUIRE_PTR(out, 16);
    const size_t need = mla_layer_workspace_size(dims, hidden, q_rank, total_tokens, nseq);
    if (!workspace || workspace_bytes < need)
      return fail(MLA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                  workspace ? workspace_bytes : static_cast<size_t>(0));
    if (!aligned(workspace, 16)) return fail(MLA_ERR_INVALID, "workspace is not 16-byte aligned");
  }
  hipError_t e = hipSuccess;
  if (total_tokens == 0) {
    if (!accumulate) {
      e = mla::launch_fill(max_logit, s.H, -INFINITY, stream);
      if (e != hipSuccess) return hip_fail(e, "max_logit init");
    }
    return MLA_OK;
  }
  e = mla::launch_layer_bf16(s.H, s.scale, hidden, q_rank, eps, x, w_dq, g_q, w_uq, w_kv_a, g_kv, w_kv_b, w_g, w_o,
                             cu_seqlens, nseq, total_tokens, out, max_logit, !accumulate, workspace, stream);
  if (e != hipSuccess) return hip_fail(e, "mla_layer_forward launch");
  return MLA_OK;
}

size_t mla_prefill_backward_workspace_size(const mla_dims* dims, int64_t total_tokens, int32_t nseq) {
  Shape s;
  if (check_dims(dims, MLA_BF16, &s) != MLA_OK || total_tokens < 0 || total_tokens > (int64_t{1} << 20) || nseq < 0)
    return 0;
  return mla::backward_ws_layout(s.H, total_tokens, nseq).total;
}

mla_status mla_prefill_backward(const mla_dims* dims, const void* q, const void* ckv, const void* ks,
                                const void* w_kv_b, const void* gate, const int32_t* cu_seqlens, int32_t nseq,
                                int64_t total_tokens, const float* out, const float* lse, const float* dout,
                                float* dq, float* dckv, float* dks, float* dw_kv_b, float* dgate, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  g_last_error.clear();
  Shape s;
  mla_status st = check_dims(dims, MLA_BF16, &s);
  if (st != MLA_OK) return st;
  if (nseq < 0 || total_tokens < 0) return fail(MLA_ERR_INVALID, "nseq and total_tokens must be >= 0");
  if (total_tokens > (int64_t{1} << 20)) return fail(MLA_ERR_UNSUPPORTED, "total_tokens above 2^20");
  if (total_tokens == 0) return MLA_OK;
  if (nseq < 1) return fail(MLA_ERR_INVALID, "total_tokens > 0 needs nseq >= 1");
  REQUIRE_PTR(cu_seqlens, 4);
  REQUIRE_PTR(q, 16);
  REQUIRE_PTR(ckv, 16);
  REQUIRE_PTR(ks, 16);
  REQUIRE_PTR(w_kv_b, 16);
  OPTIONAL_PTR(gate, 16);
  REQUIRE_PTR(out, 16);
  REQUIRE_PTR(lse, 16);
  REQUIRE_PTR(dout, 16);
  REQUIRE_PTR(dq, 16);
  REQUIRE_PTR(dckv, 16);
  REQUIRE_PTR(dks, 16);
  REQUIRE_PTR(dw_kv_b, 16);
  if (gate) REQUIRE_PTR(dgate, 16);
  const size_t need = mla_prefill_backward_workspace_size(dims, total_tokens, nseq);
  if (!workspace || workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : static_cast<size_t>(0));
  if (!aligned(workspace, 16)) return fail(MLA_ERR_INVALID, "workspace is not 16-byte aligned");
  const hipError_t e = mla::launch_prefill_backward_bf16(s.H, s.scale, q, ckv, ks, w_kv_b, gate, cu_seqlens, nseq,
                                                         total_tokens, out, lse, dout, dq, dckv, dks, dw_kv_b,
                                                         gate ? dgate : nullptr, workspace, stream);
  if (e != hipSuccess) return hip_fail(e, "mla_prefill_backward launch");
  return MLA_OK;
}

mla_status mla_qk_clip(const mla_dims* dims, mla_dtype wdtype, void* w_q_b, int32_t q_in, void* w_kv_b,
                       const float* max_logit, float tau, uint8_t* clipped, float* gamma, hipStream_t stream) {
  g_last_error.clear();
  if (!dims) return fail(MLA_ERR_INVALID, "dims is NULL");
  if (dims->heads < 1 || dims->kv_rank < 1 || dims->shared_dim < 0 || dims->nope_dim < 1 || dims->v_dim < 1)
    return fail(MLA_ERR_INVALID, "dims must be positive");
  if (wdtype != MLA_F32 && wdtype != MLA_BF16) return fail(MLA_ERR_INVALID, "unknown wdtype");
  if (!(tau > 0.0f) || !isfinite(tau)) return fail(MLA_ERR_INVALID, "tau must be finite and > 0");
  if (q_in < 1) return fail(MLA_ERR_INVALID, "q_in must be >= 1");
  const int vec = wdtype == MLA_BF16 ? 8 : 1;
  if (q_in % vec != 0 || dims->kv_rank % vec != 0)
    return fail(MLA_ERR_UNSUPPORTED, "bf16 rows must be a multiple of 8 elements (q_in=%d kv_rank=%d)", q_in,
                dims->kv_rank);
  REQUIRE_PTR(w_q_b, 16);
  REQUIRE_PTR(w_kv_b, 16);
  REQUIRE_PTR(max_logit, 4);
  OPTIONAL_PTR(gamma, 4);
  hipError_t e = mla::launch_qk_clip(dims->heads, dims->shared_dim, dims->nope_dim, dims->v_dim,
                                     wdtype == MLA_BF16, w_q_b, q_in, dims->kv_rank, w_kv_b, max_logit, tau,
                                     clipped, gamma, stream);
  if (e != hipSuccess) return hip_fail(e, "mla_qk_clip launch");
  return MLA_OK;
}

}  // extern "C"
