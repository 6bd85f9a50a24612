// Training-form gated MLA prefill in fp32 (any R <= 1024, N + S <= 256,
// V <= 256). Same equations as the bf16 path ("Kimi K3 · Gated MLA ·
// OpenModelAtlas" equation list), computed with fp32 vector arithmetic: the
// expansion writes K^C_h and V_h in fp32, then one wavefront per (query,
// head) runs the causal online softmax with the feature dimension across its
// lanes.
#include "mla_common.h"
#include "mla_internal.h"
#include "timing.h"

namespace mla {

// kcv[h][t][c], c < N: K^C_h, c >= N: V_h  =  sum_r ckv[t][r] * w[h*(N+V) + c][r]
__global__ void __launch_bounds__(256) prefill_expand_f32_kernel(const float* __restrict__ ckv,
                                                                 const float* __restrict__ w, int64_t ntok,
                                                                 int heads, int R, int NV,
                                                                 float* __restrict__ kcv) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = ntok * heads * NV;
  if (idx >= total) return;
  const int c = static_cast<int>(idx % NV);
  const int64_t rest = idx / NV;
  const int h = static_cast<int>(rest % heads);
  const int64_t t = rest / heads;
  const float* x = ckv + t * R;
  const float* wr = w + (static_cast<int64_t>(h) * NV + c) * R;
  float acc = 0.0f;
  for (int r = 0; r < R; ++r) acc = fmaf(x[r], wr[r], acc);
  kcv[(static_cast<int64_t>(h) * ntok + t) * NV + c] = acc;
}

constexpr int kF32MaxD = 256;  // N + S
constexpr int kF32MaxV = 256;

// One wavefront per (token, head); lanes hold features d = lane + 64 j.
__global__ void __launch_bounds__(256) prefill_attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ ks, const float* __restrict__ gate,
    const int32_t* __restrict__ cu, int nseq, int64_t ntok, int heads, int S, int N, int V,
    const float* __restrict__ kcv, float scale, float* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ max_logit, int qnorm, const float* __restrict__ qn_w, float qn_eps) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  if (wid >= ntok * heads) return;
  const int h = static_cast<int>(wid % heads);
  const int64_t t = wid / heads;
  int lo = 0, hi = nseq - 1;          // the sequence holding token t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int64_t a = cu[lo];
  const int D = N + S, NV = N + V;
  float qv[kF32MaxD / 64];
#pragma unroll
  for (int j = 0; j < kF32MaxD / 64; ++j) {
    const int d = lane + 64 * j;
    qv[j] = d < D ? q[(t * heads + h) * D + d] : 0.0f;
  }
  if (qnorm) {
    // QK-norm variant: the head's query over its D features divided by their
    // root mean square, times the per-feature weight
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < kF32MaxD / 64; ++j) ss = fmaf(qv[j], qv[j], ss);
    const float r = 1.0f / sqrtf(wave_sum(ss) / static_cast<float>(D) + qn_eps);
#pragma unroll
    for (int j = 0; j < kF32MaxD / 64; ++j) {
      const int d = lane + 64 * j;
      if (d < D) qv[j] = qv[j] * r * (qn_w ? qn_w[d] : 1.0f);
    }
  }
  float o[kF32MaxV / 64];
#pragma unroll
  for (int j = 0; j < kF32MaxV / 64; ++j) o[j] = 0.0f;
  float m = -INFINITY, l = 0.0f;
  const float* kh = kcv + static_cast<int64_t>(h) * ntok * NV;
  for (int64_t s = a; s <= t; ++s) {
    float part = 0.0f;
#pragma unroll
    for (int j = 0; j < kF32MaxD / 64; ++j) {
      const int d = lane + 64 * j;
      if (d < N) part = fmaf(qv[j], kh[s * NV + d], part);
      else if (d < D) part = fmaf(qv[j], ks[s * S + (d - N)], part);
    }
    const float sc = wave_sum(part) * scale;
    const float m_new = fmaxf(m, sc);
    const float corr = expf(m - m_new);
    const float p = expf(sc - m_new);
    l = l * corr + p;
#pragma unroll
    for (int j = 0; j < kF32MaxV / 64; ++j) {
      const int d = lane + 64 * j;
      o[j] = o[j] * corr + (d < V ? p * kh[s * NV + N + d] : 0.0f);
    }
    m = m_new;
  }
  const float inv = 1.0f / l;
#pragma unroll
  for (int j = 0; j < kF32MaxV / 64; ++j) {
    const int d = lane + 64 * j;
    if (d < V) {
      float v = o[j] * inv;
      if (gate) v *= 1.0f / (1.0f + expf(-gate[(t * heads + h) * V + d]));
      out[(t * heads + h) * V + d] = v;
    }
  }
  if (lane == 0) {
    if (lse) lse[static_cast<int64_t>(h) * ntok + t] = m + logf(l);
    atomic_max_float(max_logit + h, m);
  }
}

hipError_t launch_prefill_f32(int heads, int R, int S, int N, int V, float scale, const float* q,
                              const float* ckv, const float* ks, const float* w_kv_b, const float* gate,
                              const int32_t* cu, int nseq, int64_t ntok, float* out, float* lse,
                              float* max_logit, void* ws, hipStream_t st, const QNorm& qn) {
  float* kcv = static_cast<float*>(ws);
  const int NV = N + V;
  const int64_t n1 = ntok * heads * NV;
  {
    TimedScope ts_("prefill_expand_f32", st);
    hipLaunchKernelGGL(prefill_expand_f32_kernel, dim3(static_cast<unsigned>((n1 + 255) / 256)), dim3(256), 0,
                       st, ckv, w_kv_b, ntok, heads, R, NV, kcv);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t waves = ntok * heads;
  {
    TimedScope ts_("prefill_attn_f32", st);
    hipLaunchKernelGGL(prefill_attn_f32_kernel, dim3(static_cast<unsigned>((waves + 3) / 4)), dim3(256), 0, st,
                       q, ks, gate, cu, nseq, ntok, heads, S, N, V, kcv, scale, out, lse, max_logit, qn.on ? 1 : 0,
                       static_cast<const float*>(qn.w), qn.eps);
  }
  return hipGetLastError();
}

__global__ void fill_f32_kernel(float* p, int n, float v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill(float* p, int n, float v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  {
    TimedScope ts_("fill", st);
    hipLaunchKernelGGL(fill_f32_kernel, dim3((n + 255) / 256), dim3(256), 0, st, p, n, v);
  }
  return hipGetLastError();
}

}  // namespace mla
