// QK-Clip weight rescale ("SOTA-131" practice page: after a step, every head
// whose maximum attention logit exceeds the threshold tau has its query and
// key projection weights rescaled so that it no longer does).
//
// gamma_h = tau / S_max[h] for S_max[h] > tau. Each logit of head h is
// q^C_h . K^C_h + q^R_h . k^S; k^S is one vector shared by every head and is
// not touched, so the q^R rows take gamma_h and the two head-specific nope
// factors take sqrt(gamma_h) each. Unclipped heads are never written.
#include "mla_common.h"
#include "mla_internal.h"
#include "timing.h"

namespace mla {

template <bool BF16>
__global__ void __launch_bounds__(256) qk_clip_kernel(int heads, int S, int N, int V, void* __restrict__ wq,
                                                      int q_in, int R, void* __restrict__ wkv,
                                                      const float* __restrict__ max_logit, float tau,
                                                      uint8_t* __restrict__ clipped, float* __restrict__ gamma) {
  const int D = N + S;
  const int64_t row = blockIdx.x;
  const int64_t qrows = static_cast<int64_t>(heads) * D;
  int h, len;
  bool full;        // factor gamma (q^R rows) instead of sqrt(gamma)
  int64_t offset;   // element offset of the row
  void* base;
  if (row < qrows) {
    h = static_cast<int>(row / D);
    const int local = static_cast<int>(row - static_cast<int64_t>(h) * D);
    full = local >= N;
    base = wq;
    offset = row * q_in;
    len = q_in;
  } else {
    const int64_t r2 = row - qrows;
    h = static_cast<int>(r2 / N);
    const int local = static_cast<int>(r2 - static_cast<int64_t>(h) * N);
    full = false;
    base = wkv;
    offset = (static_cast<int64_t>(h) * (N + V) + local) * R;
    len = R;
  }
  const float sm = max_logit[h];
  const bool clip = sm > tau;   // strict; NaN never clips
  const float gm = clip ? tau / sm : 1.0f;
  if (row < heads && threadIdx.x == 0) {
    const float smr = max_logit[row];
    const bool c = smr > tau;
    if (clipped) clipped[row] = c ? 1 : 0;
    if (gamma) gamma[row] = c ? tau / smr : 1.0f;
  }
  if (!clip) return;
  const float f = full ? gm : sqrtf(gm);
  if (BF16) {
    uint16_t* w = static_cast<uint16_t*>(base) + offset;
    for (int i = threadIdx.x * 8; i < len; i += 256 * 8) {
      uint4 v = *reinterpret_cast<uint4*>(w + i);
      uint32_t* x = &v.x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = pack_bf16x2(bf16lo(x[e]) * f, bf16hi(x[e]) * f);
      *reinterpret_cast<uint4*>(w + i) = v;
    }
  } else {
    float* w = static_cast<float*>(base) + offset;
    for (int i = threadIdx.x; i < len; i += 256) w[i] *= f;
  }
}

hipError_t launch_qk_clip(int heads, int S, int N, int V, bool bf16, void* w_q_b, int q_in, int R, void* w_kv_b,
                          const float* max_logit, float tau, uint8_t* clipped, float* gamma, hipStream_t st) {
  const int64_t rows = static_cast<int64_t>(heads) * (N + S) + static_cast<int64_t>(heads) * N;
  if (rows > 0x7fffffff) return hipErrorInvalidValue;
  if (bf16) {
    {
      TimedScope ts_("qk_clip", st);
      hipLaunchKernelGGL(qk_clip_kernel<true>, dim3(static_cast<unsigned>(rows)), dim3(256), 0, st, heads, S, N, V,
                         w_q_b, q_in, R, w_kv_b, max_logit, tau, clipped, gamma);
    }
  } else {
    {
      TimedScope ts_("qk_clip", st);
      hipLaunchKernelGGL(qk_clip_kernel<false>, dim3(static_cast<unsigned>(rows)), dim3(256), 0, st, heads, S, N, V,
                         w_q_b, q_in, R, w_kv_b, max_logit, tau, clipped, gamma);
    }
  }
  return hipGetLastError();
}

}  // namespace mla
