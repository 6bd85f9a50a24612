// Expanded-cache decode (bf16): gated MLA attention for the last Tq positions
// of each sequence, read from a cache that keeps every token's per-head key
// K_h = [K^C_h, k^S] and value V_h, as the training form materialises them
// ("Kimi K3 · Gated MLA · OpenModelAtlas", equation list: [k^C v] = c^KV
// W_UKV, K_h = [K^C_h k^S], scaled causal softmax, O~ = A V, o = sigma(g) . o~).
// It is the per-head cache that the latent cache row of "Gated MLA et NoPE"
// (512 + 64 values per token) replaces, and serves as its bandwidth
// comparator: per token it reads H * (192 + 128) * 2 = 61,440 bytes against
// the latent row's 1,152.
//
// The work is memory-bound (one multiply-add per byte), so it runs on the
// vector ALUs and is laid out for the memory system, not for the matrix cores:
//  - Split kernel: one wave per (query, head, 2048-row split). Eight lanes
//    share a cache row: lane (g, c) = (lane / 8, lane % 8) holds 16-byte units
//    c, c+8, c+16 of the K row (192 bf16 = 24 units) and c, c+8 of the V row
//    (16 units), so each 16-byte load instruction of the wave covers eight
//    whole 128-byte lines. A pass covers 8 rows; four passes are loaded
//    together, as nontemporal loads. The score of a row is the sum over its
//    eight lanes (three DPP steps). Every lane keeps an online softmax (max,
//    sum, 16 output values) over the rows of its row group; the eight groups
//    are merged at the end and the partial (max, sum, 128 unnormalised
//    outputs) is written.
//  - Combine kernel: per (query, head), the log-sum-exp merge of the splits,
//    then the sigmoid gate.
// The per-head maximum logit is the maximum of the fp32 scores, one atomic
// per wave.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "mla_common.h"
#include "mla_internal.h"
#include "timing.h"

namespace mla {

namespace {

constexpr int kKU = kD / 8;   // 16-byte units per K row (24)
constexpr int kVU = kV / 8;   // 16-byte units per V row (16)
constexpr int kKUL = kKU / 8;  // K units per lane (3)
constexpr int kVUL = kVU / 8;  // V units per lane (2)
constexpr int kPass = 4;       // 8-row passes loaded together

// Cache rows are read once: nontemporal loads keep them from displacing
// reusable lines in the caches.
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ldg16_stream(const uint16_t* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p)));
}

// Sum over the eight lanes of an aligned group (xor 1, xor 2 inside a quad,
// then the other quad of the 8 through the half-row mirror).
__device__ __forceinline__ float sum8(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
  return x;
}

__device__ __forceinline__ float dot8(uint4 a, uint4 b, float s) {
  const bf16x8 x = __builtin_bit_cast(bf16x8, a), y = __builtin_bit_cast(bf16x8, b);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1), __builtin_shufflevector(y, y, 0, 1), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3), __builtin_shufflevector(y, y, 2, 3), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5), __builtin_shufflevector(y, y, 4, 5), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7), __builtin_shufflevector(y, y, 6, 7), s, false);
  return s;
}

// Number of splits of query i of sequence b: its visible rows lens[b] - tq + i + 1
// in pieces of kExpSplitRows.
__device__ __forceinline__ int visible_rows(const int32_t* lens, int tq, int64_t v) {
  const int64_t b = v / tq;
  const int i = static_cast<int>(v - b * tq);
  return lens[b] - tq + i + 1;
}

__global__ void __launch_bounds__(256) expanded_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kcache, const uint16_t* __restrict__ vcache,
    int64_t cap, const int32_t* __restrict__ lens, int tq, int heads, int hgroups, int smax, float scale,
    float* __restrict__ part_o, float* __restrict__ part_ml, float* __restrict__ max_logit) {
  const int64_t v = blockIdx.x / hgroups;
  const int hg = static_cast<int>(blockIdx.x - v * hgroups);
  const int split = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int h = 4 * hg + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (h >= heads) return;
  const int vis = visible_rows(lens, tq, v);
  const int r0 = split * kExpSplitRows;
  if (r0 >= vis) return;
  const int r1 = min(vis, r0 + kExpSplitRows);
  const int64_t b = v / tq;
  const int g = lane >> 3, c = lane & 7;

  // this lane's query units (the same 8 features of every row it reads)
  uint4 qu[kKUL];
  const uint16_t* qrow = q + (v * heads + h) * kD;
#pragma unroll
  for (int u = 0; u < kKUL; ++u) qu[u] = ldg16(qrow + 8 * (c + 8 * u));

  const uint16_t* kbase = kcache + ((b * heads + h) * cap) * kD + 8 * c;
  const uint16_t* vbase = vcache + ((b * heads + h) * cap) * kV + 8 * c;
  const float c2 = scale * kLog2e;

  float m = -INFINITY, l = 0.0f, mx = -INFINITY;
  float o[8 * kVUL];
#pragma unroll
  for (int e = 0; e < 8 * kVUL; ++e) o[e] = 0.0f;

  for (int base = r0; base < r1; base += 8 * kPass) {
    uint4 kr[kPass][kKUL], vr[kPass][kVUL];
#pragma unroll
    for (int k = 0; k < kPass; ++k) {
      const int j = min(base + 8 * k + g, r1 - 1);   // rows past the split repeat its last row, then are masked
#pragma unroll
      for (int u = 0; u < kKUL; ++u) kr[k][u] = ldg16_stream(kbase + static_cast<int64_t>(j) * kD + 64 * u);
#pragma unroll
      for (int u = 0; u < kVUL; ++u) vr[k][u] = ldg16_stream(vbase + static_cast<int64_t>(j) * kV + 64 * u);
    }
    float s[kPass];
    float mb = -INFINITY;
#pragma unroll
    for (int k = 0; k < kPass; ++k) {
      float d = 0.0f;
#pragma unroll
      for (int u = 0; u < kKUL; ++u) d = dot8(qu[u], kr[k][u], d);
      d = sum8(d);
      const bool valid = base + 8 * k + g < r1;
      mx = valid ? fmaxf(mx, d) : mx;
      s[k] = valid ? d * c2 : -INFINITY;
      mb = fmaxf(mb, s[k]);
    }
    const float mn = fmaxf(m, mb);
    const float ms = mn == -INFINITY ? 0.0f : mn;   // no visible row yet: every weight below is 0
    const float alpha = fast_exp2(m - ms);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < 8 * kVUL; ++e) o[e] *= alpha;
#pragma unroll
    for (int k = 0; k < kPass; ++k) {
      const float p = fast_exp2(s[k] - ms);
      l += p;
#pragma unroll
      for (int u = 0; u < kVUL; ++u) {
        const uint32_t* w = &vr[k][u].x;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[8 * u + 2 * e] = fmaf(p, bf16lo(w[e]), o[8 * u + 2 * e]);
          o[8 * u + 2 * e + 1] = fmaf(p, bf16hi(w[e]), o[8 * u + 2 * e + 1]);
        }
      }
    }
    m = mn;
  }

  // merge the eight row groups (lanes c, c+8, ..., c+56 hold the same output units)
#pragma unroll
  for (int off = 8; off <= 32; off <<= 1) {
    const float mo = __shfl_xor(m, off, 64), lo = __shfl_xor(l, off, 64);
    const float mn = fmaxf(m, mo);
    const float ms = mn == -INFINITY ? 0.0f : mn;
    const float a = fast_exp2(m - ms), ao = fast_exp2(mo - ms);
    l = l * a + lo * ao;
#pragma unroll
    for (int e = 0; e < 8 * kVUL; ++e) o[e] = o[e] * a + __shfl_xor(o[e], off, 64) * ao;
    m = mn;
  }
  const int64_t item = (v * heads + h) * smax + split;
  if (g == 0) {
    float* dst = part_o + item * kV;
#pragma unroll
    for (int u = 0; u < kVUL; ++u) {
      *reinterpret_cast<float4*>(dst + 8 * (c + 8 * u)) = make_float4(o[8 * u], o[8 * u + 1], o[8 * u + 2], o[8 * u + 3]);
      *reinterpret_cast<float4*>(dst + 8 * (c + 8 * u) + 4) =
          make_float4(o[8 * u + 4], o[8 * u + 5], o[8 * u + 6], o[8 * u + 7]);
    }
    if (c == 0) *reinterpret_cast<float2*>(part_ml + 2 * item) = make_float2(m, l);
  }
  mx = wave_max(mx);
  if (lane == 0 && mx > -INFINITY) atomic_max_float(max_logit + h, mx * scale);
}

// One workgroup of V threads per (query, head): thread d merges output d of the splits.
template <bool kOutBf16>
__global__ void __launch_bounds__(kV) expanded_combine_kernel(const float* __restrict__ part_o,
                                                              const float* __restrict__ part_ml,
                                                              const int32_t* __restrict__ lens, int tq, int heads,
                                                              int smax, const uint16_t* __restrict__ gate,
                                                              void* __restrict__ out) {
  const int64_t v = blockIdx.x;
  const int h = blockIdx.y;
  const int d = threadIdx.x;
  const int vis = visible_rows(lens, tq, v);
  const int ns = (vis + kExpSplitRows - 1) / kExpSplitRows;
  const int64_t item0 = (v * heads + h) * smax;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, part_ml[2 * (item0 + s)]);
  const float Ms = M == -INFINITY ? 0.0f : M;
  float L = 0.0f, acc = 0.0f;
  for (int s = 0; s < ns; ++s) {
    const float w = fast_exp2(part_ml[2 * (item0 + s)] - Ms);
    L = fmaf(part_ml[2 * (item0 + s) + 1], w, L);
    acc = fmaf(part_o[(item0 + s) * kV + d], w, acc);
  }
  float r = acc / L;
  const int64_t col = (v * heads + h) * kV + d;
  if (gate) r *= sigmoidf_(bf16_to_f32(gate[col]));
  if constexpr (kOutBf16) static_cast<uint16_t*>(out)[col] = f32_to_bf16(r);
  else static_cast<float*>(out)[col] = r;
}

}  // namespace

hipError_t launch_expanded_bf16(int heads, float scale, bool out_bf16, const void* q, const void* kcache,
                                const void* vcache, int64_t cap, const int32_t* lens, int batch, int tq,
                                const void* gate, void* out, float* max_logit, void* ws, hipStream_t st) {
  const ExpandedWs L = expanded_ws_layout(heads, batch, tq, cap);
  char* base = static_cast<char*>(ws);
  float* part_o = reinterpret_cast<float*>(base + L.part_o);
  float* part_ml = reinterpret_cast<float*>(base + L.part_ml);
  const int64_t bt = static_cast<int64_t>(batch) * tq;
  const int hgroups = (heads + 3) / 4;
  {
    TimedScope ts_("expanded_split", st);
    hipLaunchKernelGGL(expanded_split_kernel, dim3(static_cast<unsigned>(bt * hgroups), L.smax), dim3(256), 0, st,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kcache),
                       static_cast<const uint16_t*>(vcache), cap, lens, tq, heads, hgroups, L.smax, scale, part_o,
                       part_ml, max_logit);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    TimedScope ts_("expanded_combine", st);
    const dim3 grid(static_cast<unsigned>(bt), heads);
    if (out_bf16)
      hipLaunchKernelGGL(expanded_combine_kernel<true>, grid, dim3(kV), 0, st, part_o, part_ml, lens, tq, heads,
                         L.smax, static_cast<const uint16_t*>(gate), out);
    else
      hipLaunchKernelGGL(expanded_combine_kernel<false>, grid, dim3(kV), 0, st, part_o, part_ml, lens, tq, heads,
                         L.smax, static_cast<const uint16_t*>(gate), out);
  }
  return hipGetLastError();
}

}  // namespace mla
