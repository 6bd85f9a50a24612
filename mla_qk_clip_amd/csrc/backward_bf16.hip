// Backward of the training-form prefill (bf16): the gradients of the
// equation list of "Kimi K3 · Gated MLA · OpenModelAtlas" (expansion
// [k^C v] = c^KV W_UKV, K_h = [K^C_h, k^S], S = Q K^T / sqrt(192), causal
// softmax, O~ = A V, o = sigma(g) . o~) with respect to q, c^KV, k^S,
// kv_b_proj.weight and the gate logits, for an upstream gradient dO of o.
//
// Per sequence (length L, padded to Lp = L rounded up to 128) and chunk of
// heads, the score and probability matrices are materialised in HBM and every
// product runs on the NT GEMM kernel (batched over the chunk's heads):
//   S = Q_h K_h^T with P = causal exp(scale S - lse) in its epilogue (P, P^T
//   in bf16; S is never stored), then dP = dO~_h V_h^T with
//   dS = scale P . (dP - D), D = rowsum(dO . o), in its epilogue (dS, dS^T)
//   dQ = dS K_h, dK = dS^T Q_h, dV = P^T dO~_h          (fp32)
// Only the causal half is formed: the S and dP products skip the 256 x 256
// tiles above the diagonal (their dS, dS^T, P^T stay unwritten), and the
// three gradient products sum only over k up to (dQ) or from (dK, dV) the
// diagonal 256-block of their rows.
// with dO~ = dO . sigma(g) and dg = dO . o . (1 - sigma(g)). Operands are bf16
// (Q and K padded from 192 to 256 features with zeros); the GEMM kernel
// needs K-contiguous rows on both sides, so the transposed operands (K_h^T,
// Q_h^T, dO~^T by a tiled transpose; P^T and dS^T by the products' epilogues)
// are written out.
// Then dK^C and dV flow back through W_UKV: dc^KV = dKV W_UKV^T-rows,
// dW = dKV^T c^KV, and the k^S part of dK sums over the heads.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "mla_common.h"
#include "mla_internal.h"
#include "timing.h"

namespace mla {

namespace {

constexpr int kBwF = 256;   // padded feature width of Q_h and K_h (192 -> 256)

// Q_h, K_h (padded to 256 features), V_h and dO~_h of one sequence and head
// chunk, rows t < Lp (zeros past L); D = rowsum(dO . o); dg for t < L.
// Grid (Lp, hc), 128 threads: thread d covers features d and 128 + d.
__global__ void __launch_bounds__(128) bw_gather_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const uint16_t* __restrict__ ks,
    const uint16_t* __restrict__ gate, const float* __restrict__ out, const float* __restrict__ dout, int heads,
    int64_t a, int L, int Lp, int h0, uint16_t* __restrict__ Qp, uint16_t* __restrict__ Kp, uint16_t* __restrict__ Vh,
    uint16_t* __restrict__ dOt, float* __restrict__ Dv, float* __restrict__ dgate) {
  __shared__ float red[2];
  const int t = blockIdx.x, hh = blockIdx.y, h = h0 + hh, d = threadIdx.x;
  const int64_t row = static_cast<int64_t>(hh) * Lp + t;
  const bool live = t < L;
  const int64_t tok = a + t;
  uint16_t q0 = 0, q1 = 0, k0 = 0, k1 = 0, v = 0, go = 0;
  float pr = 0.0f;
  if (live) {
    const uint16_t* qr = q + (tok * heads + h) * kD;
    const uint16_t* kr = kv + tok * heads * (kN + kV) + static_cast<int64_t>(h) * (kN + kV);
    q0 = qr[d];
    if (d < kD - kN) q1 = qr[kN + d];
    k0 = kr[d];
    if (d < kS) k1 = ks[tok * kS + d];
    v = kr[kN + d];
    const int64_t col = tok * heads * kV + static_cast<int64_t>(h) * kV + d;
    const float dov = dout[col], ov = out[col];
    const float sg = gate ? sigmoidf_(bf16_to_f32(gate[col])) : 1.0f;
    go = f32_to_bf16(dov * sg);
    pr = dov * ov;
    if (gate) dgate[col] = dov * ov * (1.0f - sg);
  }
  Qp[row * kBwF + d] = q0;
  Qp[row * kBwF + 128 + d] = q1;
  Kp[row * kBwF + d] = k0;
  Kp[row * kBwF + 128 + d] = k1;
  Vh[row * kV + d] = v;
  dOt[row * kV + d] = go;
  pr = wave_sum(pr);
  if ((d & 63) == 0) red[d >> 6] = pr;
  __syncthreads();
  if (d == 0) Dv[row] = red[0] + red[1];
}

// dst[b][c][r] = r < rvalid ? src[b][r][c] : 0 for r < rp, c < cols (bf16).
// 64 x 64 tiles through LDS; cols and rp multiples of 4.
__global__ void __launch_bounds__(256) bw_transpose_kernel(const uint16_t* __restrict__ src, int64_t rvalid,
                                                           int64_t rp, int cols, int64_t sstride, int64_t dstride,
                                                           uint16_t* __restrict__ dst) {
  __shared__ uint16_t tile[64][64 + 4];
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int c0 = blockIdx.y * 64;
  const int64_t bz = blockIdx.z;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const uint16_t* s = src + bz * sstride;
  uint16_t* o = dst + bz * dstride;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lr = ty + 16 * i;
    const int64_t r = r0 + lr;
    const int c = c0 + 4 * tx;
    uint2 v = make_uint2(0, 0);
    if (r < rvalid && c < cols) v = *reinterpret_cast<const uint2*>(s + r * cols + c);
    tile[lr][4 * tx] = static_cast<uint16_t>(v.x);
    tile[lr][4 * tx + 1] = static_cast<uint16_t>(v.x >> 16);
    tile[lr][4 * tx + 2] = static_cast<uint16_t>(v.y);
    tile[lr][4 * tx + 3] = static_cast<uint16_t>(v.y >> 16);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lc = ty + 16 * i;
    const int c = c0 + lc;
    const int64_t r = r0 + 4 * tx;
    if (c < cols && r < rp) {
      const uint32_t x = tile[4 * tx][lc] | (static_cast<uint32_t>(tile[4 * tx + 1][lc]) << 16);
      const uint32_t y = tile[4 * tx + 2][lc] | (static_cast<uint32_t>(tile[4 * tx + 3][lc]) << 16);
      *reinterpret_cast<uint2*>(o + static_cast<int64_t>(c) * rp + r) = make_uint2(x, y);
    }
  }
}

// dq (fp32), the K^C / V gradients into dKV (bf16, head-major columns as in
// kv_b_proj) for rows t < L of one chunk; grid (L, hc), 128 threads.
__global__ void __launch_bounds__(128) bw_scatter_kernel(const float* __restrict__ dQc, const float* __restrict__ dKc,
                                                         const float* __restrict__ dVc, int heads, int64_t a, int Lp,
                                                         int h0, float* __restrict__ dq, uint16_t* __restrict__ dKV) {
  const int t = blockIdx.x, hh = blockIdx.y, h = h0 + hh, d = threadIdx.x;
  const int64_t row = static_cast<int64_t>(hh) * Lp + t, tok = a + t;
  float* dqr = dq + (tok * heads + h) * kD;
  dqr[d] = dQc[row * kBwF + d];
  if (d < kD - kN) dqr[kN + d] = dQc[row * kBwF + kN + d];
  uint16_t* o = dKV + tok * heads * (kN + kV) + static_cast<int64_t>(h) * (kN + kV);
  o[d] = f32_to_bf16(dKc[row * kBwF + d]);
  o[kN + d] = f32_to_bf16(dVc[row * kV + d]);
}

// dk^S[t] += sum over the chunk's heads of dK_h[t][128 .. 191]; grid L, 64 threads.
__global__ void __launch_bounds__(64) bw_dks_kernel(const float* __restrict__ dKc, int hc, int64_t a, int Lp,
                                                    float* __restrict__ dks) {
  const int t = blockIdx.x, j = threadIdx.x;
  float s = 0.0f;
  for (int hh = 0; hh < hc; ++hh) s += dKc[(static_cast<int64_t>(hh) * Lp + t) * kBwF + kN + j];
  dks[(a + t) * kS + j] += s;
}

__global__ void bw_zero_kernel(float* __restrict__ p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

inline int64_t round128(int64_t x) { return (x + 127) / 128 * 128; }

}  // namespace

BackwardWs backward_ws_layout(int heads, int64_t ntok, int max_seqlen) {
  BackwardWs w{};
  const size_t T = static_cast<size_t>(ntok), Tp = static_cast<size_t>(round128(ntok));
  const size_t HW = static_cast<size_t>(heads) * (kN + kV);
  const size_t Lp = static_cast<size_t>(round128(max_seqlen));
  // heads per chunk: up to 32 (the gradient products have one or two 256-wide
  // column tiles, so the chunk's heads are what fills the CUs), with the
  // Lp x Lp planes (P, P^T, dS, dS^T, bf16) within about 16 GB
  const size_t plane = Lp * Lp * (2 + 2 + 2 + 2);
  w.hc = static_cast<int>(plane ? std::max<size_t>(1, std::min<size_t>(32, (size_t{16} << 30) / plane)) : 1);
  w.hc = std::min(w.hc, heads);
  const size_t hc = static_cast<size_t>(w.hc);
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes, 256); return o; };
  w.kv = take(T * HW * 2);
  w.wT = take(HW * kR * 2);
  w.ckvT = take(static_cast<size_t>(kR) * Tp * 2);
  w.dkv = take(T * HW * 2);
  w.dkvT = take(HW * Tp * 2);
  w.qp = take(hc * Lp * kBwF * 2);
  w.qpT = take(hc * Lp * kBwF * 2);
  w.kp = take(hc * Lp * kBwF * 2);
  w.kpT = take(hc * Lp * kBwF * 2);
  w.vh = take(hc * Lp * kV * 2);
  w.dot = take(hc * Lp * kV * 2);
  w.dotT = take(hc * Lp * kV * 2);
  w.dv = take(hc * Lp * 4);
  w.p = take(hc * Lp * Lp * 2);
  w.ds = take(hc * Lp * Lp * 2);
  w.dsT = take(hc * Lp * Lp * 2);
  w.pT = take(hc * Lp * Lp * 2);
  w.dqc = take(hc * Lp * kBwF * 4);
  w.dkc = take(hc * Lp * kBwF * 4);
  w.dvc = take(hc * Lp * kV * 4);
  w.total = off;
  return w;
}

hipError_t launch_prefill_backward_bf16(int heads, float scale, const void* q, const void* ckv, const void* ks,
                                        const void* w_kv_b, const void* gate, const int32_t* cu_host, int nseq,
                                        int64_t ntok, int max_seqlen, const float* out, const float* lse,
                                        const float* dout, float* dq, float* dckv, float* dks, float* dw,
                                        float* dgate, void* ws, hipStream_t st) {
  const BackwardWs W = backward_ws_layout(heads, ntok, max_seqlen);
  char* base = static_cast<char*>(ws);
  auto b16 = [&](size_t o) { return reinterpret_cast<uint16_t*>(base + o); };
  auto f32 = [&](size_t o) { return reinterpret_cast<float*>(base + o); };
  const int HW = heads * (kN + kV);
  const int64_t Tp = round128(ntok);
  const int T = static_cast<int>(ntok);
  hipError_t e;
#define BW_CHECK()                    \
  do {                                \
    e = hipGetLastError();            \
    if (e != hipSuccess) return e;    \
  } while (0)
  // [K^C | V] of every head: c^KV W_UKV^T-rows
  {
    const GemmSpec p{static_cast<const uint16_t*>(w_kv_b), b16(W.kv), kR, HW, 0, 0, HW};
    e = launch_gemm_bf16(false, static_cast<const uint16_t*>(ckv), kR, 0, T, kR, 1, 1, &p, "bw_expand", st);
    if (e != hipSuccess) return e;
  }
  {
    TimedScope ts_("bw_transpose", st);
    hipLaunchKernelGGL(bw_transpose_kernel, dim3((HW + 63) / 64, kR / 64, 1), dim3(256), 0, st,
                       static_cast<const uint16_t*>(w_kv_b), static_cast<int64_t>(HW), static_cast<int64_t>(HW), kR,
                       int64_t{0}, int64_t{0}, b16(W.wT));
    hipLaunchKernelGGL(bw_transpose_kernel, dim3(static_cast<unsigned>(Tp / 64), kR / 64, 1), dim3(256), 0, st,
                       static_cast<const uint16_t*>(ckv), ntok, Tp, kR, int64_t{0}, int64_t{0}, b16(W.ckvT));
  }
  BW_CHECK();
  hipLaunchKernelGGL(bw_zero_kernel, dim3(static_cast<unsigned>((ntok * kS + 255) / 256)), dim3(256), 0, st, dks,
                     ntok * kS);
  BW_CHECK();
  for (int sidx = 0; sidx < nseq; ++sidx) {
    const int64_t a = cu_host[sidx];
    const int L = cu_host[sidx + 1] - cu_host[sidx];
    if (L <= 0) continue;
    const int Lp = static_cast<int>(round128(L));
    const int64_t LL = static_cast<int64_t>(Lp) * Lp;
    for (int h0 = 0; h0 < heads; h0 += W.hc) {
      const int hc = std::min(W.hc, heads - h0);
      {
        TimedScope ts_("bw_gather", st);
        hipLaunchKernelGGL(bw_gather_kernel, dim3(Lp, hc), dim3(128), 0, st, static_cast<const uint16_t*>(q),
                           b16(W.kv), static_cast<const uint16_t*>(ks), static_cast<const uint16_t*>(gate), out, dout,
                           heads, a, L, Lp, h0, b16(W.qp), b16(W.kp), b16(W.vh), b16(W.dot), f32(W.dv), dgate);
      }
      BW_CHECK();
      {
        TimedScope ts_("bw_transpose", st);
        const dim3 g256(Lp / 64, kBwF / 64, hc), g128(Lp / 64, kV / 64, hc);
        const int64_t s256 = static_cast<int64_t>(Lp) * kBwF, s128 = static_cast<int64_t>(Lp) * kV;
        hipLaunchKernelGGL(bw_transpose_kernel, g256, dim3(256), 0, st, b16(W.qp), int64_t{Lp}, int64_t{Lp}, kBwF,
                           s256, s256, b16(W.qpT));
        hipLaunchKernelGGL(bw_transpose_kernel, g256, dim3(256), 0, st, b16(W.kp), int64_t{Lp}, int64_t{Lp}, kBwF,
                           s256, s256, b16(W.kpT));
        hipLaunchKernelGGL(bw_transpose_kernel, g128, dim3(256), 0, st, b16(W.dot), int64_t{Lp}, int64_t{Lp}, kV,
                           s128, s128, b16(W.dotT));
      }
      BW_CHECK();
      {  // S = Q_h K_h^T with P = causal exp(scale S - lse) in its epilogue: P, P^T (bf16)
        const GemmSpec ps{b16(W.kp), b16(W.p), kBwF, Lp, static_cast<int64_t>(Lp) * kBwF, LL, Lp};
        const GemmSoftmaxBwd smp{kGemmEpiP, nullptr, lse, nullptr, nullptr, b16(W.pT), LL, ntok, a, h0, L, scale};
        e = launch_gemm_bf16(false, b16(W.qp), kBwF, static_cast<int64_t>(Lp) * kBwF, Lp, kBwF, hc, 1, &ps,
                             "bw_scores", st, kGemmSkipUpper, &smp);
        if (e != hipSuccess) return e;
        // dP = dO~_h V_h^T with dS = scale P (dP - D) in its epilogue: dS, dS^T (bf16)
        const GemmSpec pd{b16(W.vh), b16(W.ds), kV, Lp, static_cast<int64_t>(Lp) * kV, LL, Lp};
        const GemmSoftmaxBwd sm{kGemmEpiDS, b16(W.p), nullptr, f32(W.dv), b16(W.dsT), nullptr, LL, ntok, a, h0, L,
                                scale};
        e = launch_gemm_bf16(false, b16(W.dot), kV, static_cast<int64_t>(Lp) * kV, Lp, kV, hc, 1, &pd, "bw_dp_softmax",
                             st, kGemmSkipUpper, &sm);
        if (e != hipSuccess) return e;
      }
      {  // dQ = dS K_h, dK = dS^T Q_h, dV = P^T dO~_h (fp32)
        const GemmSpec pq{b16(W.kpT), f32(W.dqc), Lp, kBwF, static_cast<int64_t>(kBwF) * Lp,
                          static_cast<int64_t>(Lp) * kBwF, kBwF};
        e = launch_gemm_bf16(true, b16(W.ds), Lp, LL, Lp, Lp, hc, 1, &pq, "bw_grads", st, kGemmKToRow);
        if (e != hipSuccess) return e;
        const GemmSpec pk{b16(W.qpT), f32(W.dkc), Lp, kBwF, static_cast<int64_t>(kBwF) * Lp,
                          static_cast<int64_t>(Lp) * kBwF, kBwF};
        e = launch_gemm_bf16(true, b16(W.dsT), Lp, LL, Lp, Lp, hc, 1, &pk, "bw_grads", st, kGemmKFromRow);
        if (e != hipSuccess) return e;
        const GemmSpec pv{b16(W.dotT), f32(W.dvc), Lp, kV, static_cast<int64_t>(kV) * Lp,
                          static_cast<int64_t>(Lp) * kV, kV};
        e = launch_gemm_bf16(true, b16(W.pT), Lp, LL, Lp, Lp, hc, 1, &pv, "bw_grads", st, kGemmKFromRow);
        if (e != hipSuccess) return e;
      }
      {
        TimedScope ts_("bw_scatter", st);
        hipLaunchKernelGGL(bw_scatter_kernel, dim3(L, hc), dim3(128), 0, st, f32(W.dqc), f32(W.dkc), f32(W.dvc),
                           heads, a, Lp, h0, dq, b16(W.dkv));
        hipLaunchKernelGGL(bw_dks_kernel, dim3(L), dim3(64), 0, st, f32(W.dkc), hc, a, Lp, dks);
      }
      BW_CHECK();
    }
  }
  {
    TimedScope ts_("bw_transpose", st);
    hipLaunchKernelGGL(bw_transpose_kernel, dim3(static_cast<unsigned>(Tp / 64), (HW + 63) / 64, 1), dim3(256), 0,
                       st, b16(W.dkv), ntok, Tp, HW, int64_t{0}, int64_t{0}, b16(W.dkvT));
  }
  BW_CHECK();
  {  // dc^KV = dKV W_UKV (through W^T rows) and dW = dKV^T c^KV (fp32)
    const GemmSpec pc{b16(W.wT), dckv, HW, kR, 0, 0, kR};
    e = launch_gemm_bf16(true, b16(W.dkv), HW, 0, T, HW, 1, 1, &pc, "bw_weights", st);
    if (e != hipSuccess) return e;
    const GemmSpec pw{b16(W.ckvT), dw, Tp, kR, 0, 0, kR};
    e = launch_gemm_bf16(true, b16(W.dkvT), Tp, 0, HW, static_cast<int>(Tp), 1, 1, &pw, "bw_weights", st);
    if (e != hipSuccess) return e;
  }
#undef BW_CHECK
  return hipSuccess;
}

}  // namespace mla
