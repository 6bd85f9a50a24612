// Absorbed-form gated MLA in fp32 (any R <= 1024, N + S <= 256, V <= 256).
// The K up-projection is folded into the query ("Kimi Qkclip": the inference
// form skips it) and W_UV is applied to the softmax-weighted latent:
//   q~_h = W_UK_h q^C_h, s_j = scale * ([q~_h, q^R_h] . [c^KV_j, k^S_j]),
//   O~_h = (sum_j p_j c^KV_j) W_UV_h, o = sigma(g) . O~.
// One wavefront per (query token, head), latent features across its lanes.
#include "mla_common.h"
#include "mla_internal.h"
#include "timing.h"

namespace mla {

constexpr int kAbsF32MaxR = 1024;
constexpr int kAbsF32MaxS = 256;

__global__ void __launch_bounds__(256) absorbed_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ cache, int64_t cap, const int32_t* __restrict__ lens,
    int batch, int tq, int heads, int R, int S, int N, int V, const float* __restrict__ w,
    const float* __restrict__ gate, float scale, float* __restrict__ out, float* __restrict__ max_logit,
    int qnorm, const float* __restrict__ qn_w, float qn_eps) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  if (wid >= static_cast<int64_t>(batch) * tq * heads) return;
  const int h = static_cast<int>(wid % heads);
  const int64_t bq = wid / heads;
  const int b = static_cast<int>(bq / tq);
  const int i = static_cast<int>(bq % tq);
  const int D = N + S, NV = N + V, W = R + S;
  const float* qh = q + (bq * heads + h) * D;
  const float* wk = w + static_cast<int64_t>(h) * NV * R;      // rows of W_UK_h^T
  const float* wv = wk + static_cast<int64_t>(N) * R;           // rows of W_UV_h^T

  // QK-norm variant: the query's features are multiplied by r w_k, with r the
  // inverse root mean square over the head's D features
  float r = 1.0f;
  if (qnorm) {
    float ss = 0.0f;
    for (int d = lane; d < D; d += 64) ss = fmaf(qh[d], qh[d], ss);
    r = 1.0f / sqrtf(wave_sum(ss) / static_cast<float>(D) + qn_eps);
  }
  auto qval = [&](int k) { return qnorm ? qh[k] * r * (qn_w ? qn_w[k] : 1.0f) : qh[k]; };
  float qa[kAbsF32MaxR / 64];
#pragma unroll
  for (int j = 0; j < kAbsF32MaxR / 64; ++j) qa[j] = 0.0f;
  for (int k = 0; k < N; ++k) {
    const float qk = qval(k);
#pragma unroll
    for (int j = 0; j < kAbsF32MaxR / 64; ++j) {
      const int r = lane + 64 * j;
      if (r < R) qa[j] = fmaf(wk[static_cast<int64_t>(k) * R + r], qk, qa[j]);
    }
  }
  float qr[kAbsF32MaxS / 64];
#pragma unroll
  for (int j = 0; j < kAbsF32MaxS / 64; ++j) {
    const int s = lane + 64 * j;
    qr[j] = s < S ? qval(N + s) : 0.0f;
  }

  const int vis = lens[b] - tq + i + 1;
  const float* cb = cache + static_cast<int64_t>(b) * cap * W;
  float o[kAbsF32MaxR / 64];
#pragma unroll
  for (int j = 0; j < kAbsF32MaxR / 64; ++j) o[j] = 0.0f;
  float m = -INFINITY, l = 0.0f;
  for (int row = 0; row < vis; ++row) {
    const float* cr = cb + static_cast<int64_t>(row) * W;
    float part = 0.0f;
#pragma unroll
    for (int j = 0; j < kAbsF32MaxR / 64; ++j) {
      const int r = lane + 64 * j;
      if (r < R) part = fmaf(qa[j], cr[r], part);
    }
#pragma unroll
    for (int j = 0; j < kAbsF32MaxS / 64; ++j) {
      const int s = lane + 64 * j;
      if (s < S) part = fmaf(qr[j], cr[R + s], part);
    }
    const float sc = wave_sum(part) * scale;
    const float m_new = fmaxf(m, sc);
    const float corr = expf(m - m_new);
    const float p = expf(sc - m_new);
    l = l * corr + p;
#pragma unroll
    for (int j = 0; j < kAbsF32MaxR / 64; ++j) {
      const int r = lane + 64 * j;
      o[j] = o[j] * corr + (r < R ? p * cr[r] : 0.0f);
    }
    m = m_new;
  }
  const float inv = 1.0f / l;
  for (int d = 0; d < V; ++d) {
    float part = 0.0f;
#pragma unroll
    for (int j = 0; j < kAbsF32MaxR / 64; ++j) {
      const int r = lane + 64 * j;
      if (r < R) part = fmaf(o[j], wv[static_cast<int64_t>(d) * R + r], part);
    }
    const float v = wave_sum(part) * inv;
    if (lane == 0) {
      float y = v;
      if (gate) y *= 1.0f / (1.0f + expf(-gate[(bq * heads + h) * V + d]));
      out[(bq * heads + h) * V + d] = y;
    }
  }
  if (lane == 0) atomic_max_float(max_logit + h, m);
}

hipError_t launch_absorbed_f32(int heads, int R, int S, int N, int V, float scale, const float* q,
                               const float* cache, int64_t cap, const int32_t* lens, int batch, int tq,
                               const float* w_kv_b, const float* gate, float* out, float* max_logit,
                               hipStream_t st, const QNorm& qn) {
  const int64_t waves = static_cast<int64_t>(batch) * tq * heads;
  {
    TimedScope ts_("absorbed_f32", st);
    hipLaunchKernelGGL(absorbed_f32_kernel, dim3(static_cast<unsigned>((waves + 3) / 4)), dim3(256), 0, st, q,
                       cache, cap, lens, batch, tq, heads, R, S, N, V, w_kv_b, gate, scale, out, max_logit,
                       qn.on ? 1 : 0, static_cast<const float*>(qn.w), qn.eps);
  }
  return hipGetLastError();
}

}  // namespace mla
