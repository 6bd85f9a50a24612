// Absorbed-form (inference) gated MLA, bf16, Kimi K3 head shape, gfx950 MFMA.
//
// The cache holds one row [c^KV (512) | k^S (64)] per token ("Gated MLA et
// NoPE": 512 + 64 values instead of 2 x 96 x 128). The K up-projection is
// folded into the queries and W_UV is applied after the softmax ("Kimi
// Qkclip": at inference the projection is skipped):
//   q_abs_h = [W_UK_h q^C_h, q^R_h]                       (absorb kernel)
//   s_j = scale * q_abs_h . row_j,  o_lat = sum_j p_j c^KV_j  (split kernel)
//   O~_h = o_lat W_UV_h,  o = sigma(g) . O~                 (combine kernel)
//
// The split kernel is a split-K stream over the concatenation of all
// sequences' visible rows: workgroup w owns the row range [T*w/G, T*(w+1)/G)
// (T = all visible rows, G workgroups), so every workgroup reads the same
// number of cache bytes whatever the length mix. For every (workgroup,
// sequence) overlap it writes a partial (row max, denominator, unnormalised
// o_lat) for all heads; the combine kernel merges them by log-sum-exp.
#include "mla_common.h"
#include "mla_internal.h"
#include "timing.h"

namespace mla {

constexpr int kW = kR + kS;  // 576 values per cache row

// P[v] = sum of visible rows of the virtual sequences before v; virtual
// sequence v = b * tq + i sees rows 0 .. lens[b] - tq + i of cache[b].
__global__ void __launch_bounds__(64) absorbed_prefix_kernel(const int32_t* __restrict__ lens, int batch, int tq,
                                                             int64_t* __restrict__ P) {
  if (threadIdx.x != 0) return;
  int64_t acc = 0;
  for (int b = 0; b < batch; ++b)
    for (int i = 0; i < tq; ++i) {
      P[static_cast<int64_t>(b) * tq + i] = acc;
      acc += lens[b] - tq + i + 1;
    }
  P[static_cast<int64_t>(batch) * tq] = acc;
}

// q_abs[v][h][r] = sum_k w_kv_b[h*256 + k][r] * q[v][h][k]  (r < 512),
// q_abs[v][h][512 + s] = q[v][h][128 + s].  Grid (heads, 2): 256 columns r per block.
constexpr int kAbsQChunk = 32;
__global__ void __launch_bounds__(256) absorb_q_kernel(const uint16_t* __restrict__ q,
                                                       const uint16_t* __restrict__ w, int bt, int heads,
                                                       uint16_t* __restrict__ qabs) {
  __shared__ float qc[kAbsQChunk][kN];
  const int h = blockIdx.x;
  const int r = blockIdx.y * 256 + threadIdx.x;
  const uint16_t* wk = w + static_cast<size_t>(h) * 256 * kR + r;
  for (int v0 = 0; v0 < bt; v0 += kAbsQChunk) {
    const int nv = min(kAbsQChunk, bt - v0);
    __syncthreads();
    for (int e = threadIdx.x; e < nv * kN; e += 256) {
      const int v = e / kN, k = e - v * kN;
      qc[v][k] = bf16_to_f32(q[(static_cast<size_t>(v0 + v) * heads + h) * kD + k]);
    }
    __syncthreads();
    float acc[kAbsQChunk];
#pragma unroll
    for (int v = 0; v < kAbsQChunk; ++v) acc[v] = 0.0f;
    for (int k = 0; k < kN; ++k) {
      const float wv = bf16_to_f32(wk[static_cast<size_t>(k) * kR]);
#pragma unroll
      for (int v = 0; v < kAbsQChunk; ++v) acc[v] = fmaf(wv, qc[v][k], acc[v]);
    }
    for (int v = 0; v < nv; ++v) qabs[(static_cast<size_t>(v0 + v) * heads + h) * kW + r] = f32_to_bf16(acc[v]);
    if (blockIdx.y == 0 && threadIdx.x < kS) {
      for (int v = 0; v < nv; ++v)
        qabs[(static_cast<size_t>(v0 + v) * heads + h) * kW + kR + threadIdx.x] =
            q[(static_cast<size_t>(v0 + v) * heads + h) * kD + kN + threadIdx.x];
    }
  }
}

// ---------------------------------------------------------------------------
// Split kernel. 4 waves; wave w < ceil(H/32) owns heads 32w .. 32w+31: it keeps
// their q_abs as MFMA operands in registers, forms S^T = C Q^T for each tile
// of 32 rows (each lane owns one head column), runs the online softmax and
// accumulates O_lat^T = C^T P^T (512 x 32) in registers. All 256 threads load
// each tile once from HBM into LDS twice: row-major (score operand) and
// transposed with the value-operand row permutation (latent operand).
// Partials: part_ml[slot][h] = {raw row max, denominator}, part_o[slot][h][r]
// = unnormalised o_lat, slot = workgroup + virtual sequence.
// ---------------------------------------------------------------------------
constexpr int kCsLd = kW + 8;            // 584
constexpr int kCtLd = kDecRows + 8;      // 40

__global__ void __launch_bounds__(256) absorbed_split_kernel(
    const uint16_t* __restrict__ cache, int64_t cap, int tq, int heads, int64_t bt,
    const int64_t* __restrict__ P, const uint16_t* __restrict__ qabs, float scale,
    float* __restrict__ part_o, float* __restrict__ part_ml) {
  __shared__ __align__(16) uint16_t Cs[kDecRows * kCsLd];
  __shared__ __align__(16) uint16_t Ct[kR * kCtLd];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int G = gridDim.x;
  const int64_t total = P[bt];
  int64_t lo = total * blockIdx.x / G;
  const int64_t hi = total * (blockIdx.x + 1) / G;
  if (lo >= hi) return;

  const int head = 32 * wave + l32;
  const bool hvalid = head < heads;
  const bool active = 32 * wave < heads;   // this wave owns some heads
  const float c2 = scale * kLog2e;

  // virtual sequence holding row lo
  int64_t vlo = 0, vhi = bt - 1;
  while (vlo < vhi) {
    const int64_t mid = (vlo + vhi + 1) >> 1;
    if (P[mid] <= lo) vlo = mid; else vhi = mid - 1;
  }
  int64_t vs = vlo;

  while (lo < hi) {
    while (P[vs + 1] <= lo) ++vs;
    const int64_t seg_end = min(hi, P[vs + 1]);
    const int b = static_cast<int>(vs / tq);
    const int r0 = static_cast<int>(lo - P[vs]);
    const int r1 = static_cast<int>(seg_end - P[vs]);
    const uint16_t* cb = cache + static_cast<size_t>(b) * cap * kW;

    bf16x8 qf[kW / 16];
    {
      const uint16_t* qrow = qabs + (static_cast<size_t>(vs) * heads + (hvalid ? head : 0)) * kW + 8 * g;
#pragma unroll
      for (int kk = 0; kk < kW / 16; ++kk)
        qf[kk] = as_bf16x8(hvalid ? ldg16(qrow + 16 * kk) : make_uint4(0, 0, 0, 0));
    }
    f32x16 oacc[kR / 32];
#pragma unroll
    for (int i = 0; i < kR / 32; ++i) oacc[i] = f32x16{};
    float m_raw = -INFINITY, l_part = 0.0f;

    for (int t0 = r0; t0 < r1; t0 += kDecRows) {
      const int nrows = min(kDecRows, r1 - t0);
      // ---- load the tile as 8x8 blocks (8 rows x 8 features) ----
      __syncthreads();
      for (int blkid = tid; blkid < 4 * (kW / 8); blkid += 256) {
        const int rg = blkid / (kW / 8);
        const int dg = blkid - rg * (kW / 8);
        const int base = 16 * (rg >> 1) + 4 * (rg & 1);
        uint4 rows[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int rr = base + (e & 3) + ((e >> 2) << 3);
          rows[e] = rr < nrows ? ldg16(cb + static_cast<size_t>(t0 + rr) * kW + 8 * dg) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int rr = base + (e & 3) + ((e >> 2) << 3);
          *reinterpret_cast<uint4*>(Cs + rr * kCsLd + 8 * dg) = rows[e];
        }
        if (dg < kR / 8) {
          const int pos = 16 * (rg >> 1) + 8 * (rg & 1);
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            uint32_t wd[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const uint32_t a = (&rows[2 * k].x)[c >> 1];
              const uint32_t bb = (&rows[2 * k + 1].x)[c >> 1];
              wd[k] = (c & 1) ? ((a >> 16) | (bb & 0xffff0000u)) : ((a & 0xffffu) | (bb << 16));
            }
            *reinterpret_cast<uint4*>(Ct + (8 * dg + c) * kCtLd + pos) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
          }
        }
      }
      __syncthreads();
      if (!active) continue;

      // ---- S^T (32 rows x 32 heads), raw scores ----
      f32x16 sacc = f32x16{};
#pragma unroll
      for (int kk = 0; kk < kW / 16; ++kk) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(Cs + l32 * kCsLd + 16 * kk + 8 * g));
        sacc = mfma32(a, qf[kk], sacc);
      }
      if (nrows < kDecRows) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (acc_row(e, g) >= nrows) sacc[e] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[e]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_raw, mx);
      const float m_use = m_new == -INFINITY ? 0.0f : m_new;
      const float corr = fast_exp2((m_raw - m_use) * c2);
      const float moff = -m_use * c2;
      m_raw = m_new;
      uint32_t pk[8];
      float psum = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const float p0 = fast_exp2(fmaf(sacc[e], c2, moff));
        const float p1 = fast_exp2(fmaf(sacc[e + 1], c2, moff));
        psum += p0 + p1;
        pk[e >> 1] = pack_bf16x2(p0, p1);
      }
      l_part = l_part * corr + psum;
#pragma unroll
      for (int i = 0; i < kR / 32; ++i) oacc[i] *= corr;

      // ---- O_lat^T (512 x 32 heads) += C^T P^T ----
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const bf16x8 bp = as_bf16x8(make_uint4(pk[4 * jj], pk[4 * jj + 1], pk[4 * jj + 2], pk[4 * jj + 3]));
#pragma unroll
        for (int cbk = 0; cbk < kR / 32; ++cbk) {
          const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(Ct + (32 * cbk + l32) * kCtLd + 16 * jj + 8 * g));
          oacc[cbk] = mfma32(a, bp, oacc[cbk]);
        }
      }
    }

    // ---- partial for (this workgroup, vs) ----
    if (active && hvalid) {
      const size_t slot = static_cast<size_t>(blockIdx.x) + static_cast<size_t>(vs);
      float* po = part_o + (slot * heads + head) * kR;
#pragma unroll
      for (int cbk = 0; cbk < kR / 32; ++cbk)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          const int r = 32 * cbk + 8 * grp + 4 * g;
          *reinterpret_cast<float4*>(po + r) =
              make_float4(oacc[cbk][4 * grp], oacc[cbk][4 * grp + 1], oacc[cbk][4 * grp + 2], oacc[cbk][4 * grp + 3]);
        }
      const float l_tot = l_part + __shfl_xor(l_part, 32, 64);
      if (g == 0) {
        part_ml[(slot * heads + head) * 2] = m_raw;
        part_ml[(slot * heads + head) * 2 + 1] = l_tot;
      }
    }
    lo = seg_end;
  }
}

// ---------------------------------------------------------------------------
// Combine: merge the partials of each (virtual sequence, head) by log-sum-exp,
// then O~ = o_lat W_UV_h, gate, store, and the per-head max logit.
// Grid (heads, ceil(bt / 16)); 256 threads.
// ---------------------------------------------------------------------------
constexpr int kCmbV = 16;

__device__ __forceinline__ int split_of_row(int64_t total, int G, int64_t row) {
  // largest w with floor(total * w / G) <= row
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (total * mid / G <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <bool OUT_BF16>
__global__ void __launch_bounds__(256) absorbed_combine_kernel(
    const int64_t* __restrict__ P, int64_t bt, int G, int heads, float scale,
    const float* __restrict__ part_o, const float* __restrict__ part_ml, const uint16_t* __restrict__ w,
    const uint16_t* __restrict__ gate, void* __restrict__ out, float* __restrict__ max_logit) {
  __shared__ float olat[kCmbV][kR];
  __shared__ float red[kCmbV];
  const int h = blockIdx.x;
  const int64_t v0 = static_cast<int64_t>(blockIdx.y) * kCmbV;
  const int tid = threadIdx.x;
  const int vl = tid >> 4, sub = tid & 15;
  const int64_t vs = v0 + vl;
  const int64_t total = P[bt];
  const float c2 = scale * kLog2e;
  float mmax = -INFINITY;
  if (vs < bt) {
    const int wa = split_of_row(total, G, P[vs]);
    const int wb = split_of_row(total, G, P[vs + 1] - 1);
    float M = -INFINITY;
    for (int wg = wa; wg <= wb; ++wg) M = fmaxf(M, part_ml[((static_cast<size_t>(wg) + vs) * heads + h) * 2]);
    float den = 0.0f;
    float acc[kR / 16];
#pragma unroll
    for (int e = 0; e < kR / 16; ++e) acc[e] = 0.0f;
    for (int wg = wa; wg <= wb; ++wg) {
      const size_t s = (static_cast<size_t>(wg) + vs) * heads + h;
      const float f = fast_exp2((part_ml[s * 2] - M) * c2);
      den += f * part_ml[s * 2 + 1];
      const float* po = part_o + s * kR + sub * (kR / 16);
#pragma unroll
      for (int e = 0; e < kR / 16; e += 4) {
        const float4 x = *reinterpret_cast<const float4*>(po + e);
        acc[e] += f * x.x; acc[e + 1] += f * x.y; acc[e + 2] += f * x.z; acc[e + 3] += f * x.w;
      }
    }
    const float inv = 1.0f / den;
#pragma unroll
    for (int e = 0; e < kR / 16; ++e) olat[vl][sub * (kR / 16) + e] = acc[e] * inv;
    mmax = M;
  } else {
#pragma unroll
    for (int e = 0; e < kR / 16; ++e) olat[vl][sub * (kR / 16) + e] = 0.0f;
  }
  if (sub == 0) red[vl] = mmax;
  __syncthreads();
  if (tid == 0) {
    float mm = -INFINITY;
    for (int i = 0; i < kCmbV; ++i) mm = fmaxf(mm, red[i]);
    if (mm > -INFINITY) atomic_max_float(max_logit + h, mm * scale);
  }

  // O~[v][d] = sum_r olat[v][r] * w_kv_b[h*256 + 128 + d][r]
  const int d = tid & 127;
  const int vh = tid >> 7;   // 8 virtual sequences each
  const uint16_t* wv = w + (static_cast<size_t>(h) * 256 + kN + d) * kR;
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.0f;
  for (int r = 0; r < kR; r += 8) {
    const uint4 wq = ldg16(wv + r);
    const float wf[8] = {bf16lo(wq.x), bf16hi(wq.x), bf16lo(wq.y), bf16hi(wq.y),
                         bf16lo(wq.z), bf16hi(wq.z), bf16lo(wq.w), bf16hi(wq.w)};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float* ol = &olat[vh * 8 + i][r];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[i] = fmaf(ol[e], wf[e], o[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t v = v0 + vh * 8 + i;
    if (v >= bt) continue;
    float y = o[i];
    const size_t idx = (static_cast<size_t>(v) * heads + h) * kV + d;
    if (gate) y *= sigmoidf_(bf16_to_f32(gate[idx]));
    if (OUT_BF16) static_cast<uint16_t*>(out)[idx] = f32_to_bf16(y);
    else static_cast<float*>(out)[idx] = y;
  }
}

hipError_t launch_absorbed_bf16(int heads, float scale, bool out_bf16, const void* q, const void* cache,
                                int64_t cap, const int32_t* lens, int batch, int tq, const void* w_kv_b,
                                const void* gate, void* out, float* max_logit, void* ws, hipStream_t st) {
  const AbsorbedWs L = absorbed_ws_layout(heads, batch, tq);
  char* base = static_cast<char*>(ws);
  uint16_t* qabs = reinterpret_cast<uint16_t*>(base + L.qabs);
  int64_t* P = reinterpret_cast<int64_t*>(base + L.prefix);
  float* part_o = reinterpret_cast<float*>(base + L.part_o);
  float* part_ml = reinterpret_cast<float*>(base + L.part_ml);
  const int64_t bt = static_cast<int64_t>(batch) * tq;

  {
    TimedScope ts_("absorbed_prefix", st);
    hipLaunchKernelGGL(absorbed_prefix_kernel, dim3(1), dim3(64), 0, st, lens, batch, tq, P);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    TimedScope ts_("absorb_q", st);
    hipLaunchKernelGGL(absorb_q_kernel, dim3(heads, kR / 256), dim3(256), 0, st, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(w_kv_b), static_cast<int>(bt), heads, qabs);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    TimedScope ts_("absorbed_split", st);
    hipLaunchKernelGGL(absorbed_split_kernel, dim3(kDecSplits), dim3(256), 0, st,
                       static_cast<const uint16_t*>(cache), cap, tq, heads, bt, P, qabs, scale, part_o, part_ml);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 cg(heads, static_cast<unsigned>((bt + kCmbV - 1) / kCmbV));
  if (out_bf16) {
    {
      TimedScope ts_("absorbed_combine", st);
      hipLaunchKernelGGL(absorbed_combine_kernel<true>, cg, dim3(256), 0, st, P, bt, kDecSplits, heads, scale,
                         part_o, part_ml, static_cast<const uint16_t*>(w_kv_b),
                         static_cast<const uint16_t*>(gate), out, max_logit);
    }
  } else {
    {
      TimedScope ts_("absorbed_combine", st);
      hipLaunchKernelGGL(absorbed_combine_kernel<false>, cg, dim3(256), 0, st, P, bt, kDecSplits, heads, scale,
                         part_o, part_ml, static_cast<const uint16_t*>(w_kv_b),
                         static_cast<const uint16_t*>(gate), out, max_logit);
    }
  }
  return hipGetLastError();
}

}  // namespace mla
