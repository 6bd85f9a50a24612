// Training-form gated MLA prefill, bf16 inputs, Kimi K3 head shape
// (R = 512, S = 64, N = 128, V = 128), gfx950 MFMA.
//
// Follows the equation list of "Kimi K3 · Gated MLA · OpenModelAtlas":
//   [k^C v] = c^KV W_UKV (expansion, materialised once into the workspace),
//   K_h = [K^C_h, k^S], S = Q K^T / sqrt(192), causal softmax, O~ = A V,
//   o = sigma(g) . reshape(O~); plus the per-head maximum of S that QK-Clip
//   ("SOTA-131") needs.
//
// Three launches: a one-workgroup plan (per-sequence padded offsets and a
// longest-first tile order), the expansion GEMM, and the attention kernel.
#include "mla_common.h"
#include "mla_internal.h"
#include "timing.h"

namespace mla {

// ---------------------------------------------------------------------------
// Plan: pcu[s] = start of sequence s in the padded workspace (each sequence
// rounded up to 64 rows), order[] = sequences by descending length, toff[r] =
// first query tile of the r-th sequence in that order, hdr = {tiles, padded rows}.
// ---------------------------------------------------------------------------
constexpr int kPlanSortMax = 4096;

__global__ void __launch_bounds__(256) prefill_plan_kernel(const int32_t* __restrict__ cu, int nseq,
                                                           int32_t* __restrict__ pcu,
                                                           int32_t* __restrict__ order,
                                                           int32_t* __restrict__ toff,
                                                           int32_t* __restrict__ hdr) {
  __shared__ int s_order[kPlanSortMax];
  const bool sort = nseq <= kPlanSortMax;
  if (sort) {
    for (int s = threadIdx.x; s < nseq; s += blockDim.x) {
      const int L = cu[s + 1] - cu[s];
      int rank = 0;
      for (int t = 0; t < nseq; ++t) {
        const int Lt = cu[t + 1] - cu[t];
        rank += (Lt > L) || (Lt == L && t < s);
      }
      s_order[rank] = s;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int p = 0;
    for (int s = 0; s < nseq; ++s) {
      pcu[s] = p;
      const int L = cu[s + 1] - cu[s];
      p += (L + kSeqPad - 1) / kSeqPad * kSeqPad;
    }
    pcu[nseq] = p;
    int t = 0;
    for (int r = 0; r < nseq; ++r) {
      const int s = sort ? s_order[r] : r;
      order[r] = s;
      toff[r] = t;
      const int L = cu[s + 1] - cu[s];
      t += (L + kPrefBM - 1) / kPrefBM;
    }
    toff[nseq] = t;
    hdr[0] = t;
    hdr[1] = p;
  }
}

// ---------------------------------------------------------------------------
// Expansion: C[p, j] = sum_k c^KV[src(p), k] * w_kv_b[j, k] over padded rows p.
// One workgroup = 128 padded rows x one 128-wide half of one head (even half:
// K^C_h, odd half: V_h). K^C goes to kc[h][p][d]; V goes transposed to
// vt[h][d][p'] with p' the value-operand permutation inside each 16-row group.
// ---------------------------------------------------------------------------
constexpr int kExBM = 128, kExBN = 128, kExBK = 64, kExLd = kExBK + 8, kExOutLd = 128 + 8;

__global__ void __launch_bounds__(256) prefill_expand_kernel(
    const uint16_t* __restrict__ ckv, const uint16_t* __restrict__ w, const int32_t* __restrict__ cu,
    int nseq, const int32_t* __restrict__ pcu, const int32_t* __restrict__ hdr, int64_t npad_max,
    const uint16_t* __restrict__ ks, uint16_t* __restrict__ kc, uint16_t* __restrict__ vt,
    float* __restrict__ aux) {
  __shared__ __align__(16) uint16_t smem[2 * kExBM * kExLd];
  __shared__ int src_row[kExBM];
  __shared__ float red[4];
  static_assert(kExBM * kExOutLd <= 2 * kExBM * kExLd, "staging must fit");

  const int npad = hdr[1];
  const int m0 = blockIdx.y * kExBM;
  if (m0 >= npad) return;
  const int head = blockIdx.x >> 1, half = blockIdx.x & 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;

  if (tid < kExBM) {
    const int p = m0 + tid;
    int src = -1;
    if (p < npad) {
      int lo = 0, hi = nseq - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pcu[mid] <= p) lo = mid; else hi = mid - 1;
      }
      const int local = p - pcu[lo];
      if (local < cu[lo + 1] - cu[lo]) src = cu[lo] + local;
    }
    src_row[tid] = src;
  }
  __syncthreads();

  uint16_t* As = smem;
  uint16_t* Bs = smem + kExBM * kExLd;
  const uint16_t* wrow = w + (static_cast<size_t>(head) * 256 + half * 128) * kR;

  uint4 ra[4], rb[4];
  auto load = [&](int k0) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int id = tid + 256 * c;
      const int row = id >> 3, part = id & 7;
      const int src = src_row[row];
      ra[c] = src >= 0 ? ldg16(ckv + static_cast<size_t>(src) * kR + k0 + 8 * part) : make_uint4(0, 0, 0, 0);
      rb[c] = ldg16(wrow + static_cast<size_t>(row) * kR + k0 + 8 * part);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  load(0);
  for (int kt = 0; kt < kR / kExBK; ++kt) {
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int id = tid + 256 * c;
      const int row = id >> 3, part = id & 7;
      *reinterpret_cast<uint4*>(As + row * kExLd + 8 * part) = ra[c];
      *reinterpret_cast<uint4*>(Bs + row * kExLd + 8 * part) = rb[c];
    }
    __syncthreads();
    if (kt + 1 < kR / kExBK) load((kt + 1) * kExBK);
#pragma unroll
    for (int ks = 0; ks < kExBK / 16; ++ks) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = as_bf16x8(*reinterpret_cast<const uint4*>(As + (wm * 64 + 32 * i + l32) * kExLd + 16 * ks + 8 * g));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = as_bf16x8(*reinterpret_cast<const uint4*>(Bs + (wn * 64 + 32 * j + l32) * kExLd + 16 * ks + 8 * g));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
    }
  }

  // stage the 128 x 128 tile as bf16 in its final orientation
  __syncthreads();
  uint16_t* st = smem;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = wm * 64 + 32 * i + acc_row(e, g);   // padded row within the tile
        const int n = wn * 64 + 32 * j + l32;             // feature within the half
        const uint16_t v = f32_to_bf16(acc[i][j][e]);
        if (half == 0) st[m * kExOutLd + n] = v;
        else st[n * kExOutLd + ((m & ~15) | vperm16(m & 15))] = v;
      }
  __syncthreads();
  if (half == 0) {
    // largest squared norm of a stored K^C row (and, once, of a k^S row): the
    // error bound of the max-logit refinement
    const int row = tid >> 1, part = tid & 1;
    float n2 = 0.0f;
#pragma unroll 8
    for (int e = 0; e < 64; e += 2) {
      const uint32_t w2 = *reinterpret_cast<const uint32_t*>(st + row * kExOutLd + 64 * part + e);
      n2 = fmaf(bf16lo(w2), bf16lo(w2), fmaf(bf16hi(w2), bf16hi(w2), n2));
    }
    n2 += __shfl_xor(n2, 1, 64);
    float s2 = 0.0f;
    if (head == 0 && part == 0 && src_row[row] >= 0) {
      const uint16_t* kr = ks + static_cast<size_t>(src_row[row]) * kS;
      for (int e = 0; e < kS; e += 8) {
        const uint4 w4 = ldg16(kr + e);
        const uint32_t* x = &w4.x;
#pragma unroll
        for (int u = 0; u < 4; ++u) s2 = fmaf(bf16lo(x[u]), bf16lo(x[u]), fmaf(bf16hi(x[u]), bf16hi(x[u]), s2));
      }
    }
    n2 = wave_max(n2);
    s2 = wave_max(s2);
    if (lane == 0) red[wave] = n2;
    __syncthreads();
    if (tid == 0) atomic_max_float(aux + head * kAuxStride + 2, fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
    if (head == 0 && lane == 0) atomic_max_float(aux + static_cast<size_t>(gridDim.x / 2) * kAuxStride, s2);
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int id = tid + 256 * c;
    const int row = id >> 4, part = id & 15;
    const uint4 v = *reinterpret_cast<const uint4*>(st + row * kExOutLd + 8 * part);
    if (half == 0) {
      stg16(kc + (static_cast<size_t>(head) * npad_max + m0 + row) * kN + 8 * part, v);
    } else {
      stg16(vt + (static_cast<size_t>(head) * kV + row) * npad_max + m0 + 8 * part, v);
    }
  }
}

// ---------------------------------------------------------------------------
// Attention. One workgroup = one head x 128 queries of one sequence; 4 waves
// of 32 queries. Scores are formed transposed (S^T = K Q^T) so that each lane
// owns one query column: the row max/sum and the output rescale stay in the
// lane. Keys are visited in tiles of 64 up to the diagonal (tiles above it
// are skipped); only the diagonal tiles are masked.
// ---------------------------------------------------------------------------
constexpr int kKsLd = kD + 8;       // 200 bf16 per key row in LDS
constexpr int kVsLd = kPrefBN + 8;  // 72 bf16 per value-transposed row in LDS

template <bool OUT_BF16>
__global__ void __launch_bounds__(256) prefill_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ ks, const uint16_t* __restrict__ gate,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ pcu, const int32_t* __restrict__ order,
    const int32_t* __restrict__ toff, const int32_t* __restrict__ hdr, int nseq, int heads,
    int64_t ntok, int64_t npad_max, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vt,
    float scale, void* __restrict__ out, float* __restrict__ lse, float* __restrict__ rowmax,
    float* __restrict__ aux) {
  __shared__ __align__(16) uint16_t Ks[kPrefBN * kKsLd];
  __shared__ __align__(16) uint16_t Vs[kV * kVsLd];
  __shared__ float red[4];
  __shared__ float redq[4];

  // ---- work item: blocks that share a head run on the same XCD ----
  const int ntiles = hdr[0];
  const int total = ntiles * heads;
  const int per_xcd = (total + 7) >> 3;
  const int b = blockIdx.x;
  const int slot = b >> 3;
  if (slot >= per_xcd) return;
  const int item = (b & 7) * per_xcd + slot;
  if (item >= total) return;
  const int head = item / ntiles;
  const int tile = item - head * ntiles;
  int lo = 0, hi = nseq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (toff[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  const int seq = order[lo];
  const int a0 = cu[seq];
  const int L = cu[seq + 1] - a0;
  const int nqt = (L + kPrefBM - 1) / kPrefBM;
  const int qt = nqt - 1 - (tile - toff[lo]);   // longest tiles first
  const int pbase = pcu[seq];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int q0 = qt * kPrefBM;
  const int qi = q0 + 32 * wave + l32;           // this lane's query (sequence-local)
  const bool qvalid = qi < L;
  const int nkv = min(L, q0 + kPrefBM);
  const int nkt = (nkv + kPrefBN - 1) / kPrefBN;

  // ---- queries, held as MFMA B operands for the whole loop ----
  bf16x8 qf[kD / 16];
  {
    const uint16_t* qrow = q + (static_cast<size_t>(a0 + (qvalid ? qi : 0)) * heads + head) * kD + 8 * g;
#pragma unroll
    for (int kk = 0; kk < kD / 16; ++kk)
      qf[kk] = as_bf16x8(qvalid ? ldg16(qrow + 16 * kk) : make_uint4(0, 0, 0, 0));
  }

  const uint16_t* kc_h = kc + (static_cast<size_t>(head) * npad_max + pbase) * kN;
  const uint16_t* vt_h = vt + static_cast<size_t>(head) * kV * npad_max + pbase;

  uint4 rk[6], rv[4];
  auto load_tile = [&](int j) {
    const int kv0 = j * kPrefBN;
#pragma unroll
    for (int c = 0; c < 6; ++c) {
      const int id = tid + 256 * c;          // 64 rows x 24 chunks
      const int row = id / 24, part = id - row * 24;
      const int kv = kv0 + row;
      if (part < 16) {
        rk[c] = ldg16(kc_h + static_cast<size_t>(kv) * kN + 8 * part);
      } else {
        rk[c] = kv < L ? ldg16(ks + static_cast<size_t>(a0 + kv) * kS + 8 * (part - 16)) : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int id = tid + 256 * c;          // 128 rows x 8 chunks
      const int d = id >> 3, part = id & 7;
      rv[c] = ldg16(vt_h + static_cast<size_t>(d) * npad_max + kv0 + 8 * part);
    }
  };

  f32x16 oacc[kV / 32];
#pragma unroll
  for (int i = 0; i < kV / 32; ++i) oacc[i] = f32x16{};
  float m_raw = -INFINITY;   // running max of raw (unscaled) scores of this lane's query
  float l_part = 0.0f;       // this lane half's share of the softmax denominator
  const float c2 = scale * kLog2e;

  load_tile(0);
  for (int j = 0; j < nkt; ++j) {
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 6; ++c) {
      const int id = tid + 256 * c;
      const int row = id / 24, part = id - row * 24;
      *reinterpret_cast<uint4*>(Ks + row * kKsLd + 8 * part) = rk[c];
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int id = tid + 256 * c;
      const int d = id >> 3, part = id & 7;
      *reinterpret_cast<uint4*>(Vs + d * kVsLd + 8 * part) = rv[c];
    }
    __syncthreads();
    if (j + 1 < nkt) load_tile(j + 1);

    // S^T for the 64 keys of this tile: two 32x32 blocks
    f32x16 sacc[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      f32x16 acc = f32x16{};
#pragma unroll
      for (int kk = 0; kk < kD / 16; ++kk) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(Ks + (32 * blk + l32) * kKsLd + 16 * kk + 8 * g));
        acc = mfma32(a, qf[kk], acc);
      }
      sacc[blk] = acc;
    }

    // causal mask on the diagonal tiles
    const int kv0 = j * kPrefBN;
    if (kv0 + kPrefBN - 1 > q0 + 32 * wave) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int kv = kv0 + 32 * blk + acc_row(e, g);
          if (kv > qi) sacc[blk][e] = -INFINITY;
        }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[blk][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_raw, mx);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    const float corr = fast_exp2((m_raw - m_use) * c2);
    const float moff = -m_use * c2;
    m_raw = m_new;

    uint32_t pk[2][8];
    float psum = 0.0f;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const float p0 = fast_exp2(fmaf(sacc[blk][e], c2, moff));
        const float p1 = fast_exp2(fmaf(sacc[blk][e + 1], c2, moff));
        psum += p0 + p1;
        pk[blk][e >> 1] = pack_bf16x2(p0, p1);
      }
    l_part = l_part * corr + psum;
#pragma unroll
    for (int i = 0; i < kV / 32; ++i) oacc[i] *= corr;

    // O^T += V^T P^T, 16 keys per MFMA
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint32_t* src = &pk[jj >> 1][4 * (jj & 1)];
      const bf16x8 bp = as_bf16x8(make_uint4(src[0], src[1], src[2], src[3]));
#pragma unroll
      for (int db = 0; db < kV / 32; ++db) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(Vs + (32 * db + l32) * kVsLd + 16 * jj + 8 * g));
        oacc[db] = mfma32(a, bp, oacc[db]);
      }
    }
  }

  // ---- epilogue: normalise, gate, store; log-sum-exp; per-head max logit ----
  const float l_tot = l_part + __shfl_xor(l_part, 32, 64);
  const float inv = 1.0f / l_tot;
  if (qvalid) {
    const size_t t = static_cast<size_t>(a0 + qi);
    const uint16_t* grow = gate ? gate + (t * heads + head) * kV : nullptr;
#pragma unroll
    for (int db = 0; db < kV / 32; ++db)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const int d = 32 * db + 8 * grp + 4 * g;
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = oacc[db][4 * grp + e] * inv;
        if (grow) {
          const uint2 gv = *reinterpret_cast<const uint2*>(grow + d);
          o[0] *= sigmoidf_(bf16lo(gv.x));
          o[1] *= sigmoidf_(bf16hi(gv.x));
          o[2] *= sigmoidf_(bf16lo(gv.y));
          o[3] *= sigmoidf_(bf16hi(gv.y));
        }
        if (OUT_BF16) {
          uint16_t* orow = static_cast<uint16_t*>(out) + (t * heads + head) * kV + d;
          *reinterpret_cast<uint2*>(orow) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
        } else {
          float* orow = static_cast<float*>(out) + (t * heads + head) * kV + d;
          *reinterpret_cast<float4*>(orow) = make_float4(o[0], o[1], o[2], o[3]);
        }
      }
    if (g == 0) {
      if (lse) lse[static_cast<size_t>(head) * ntok + t] = m_raw * scale + __logf(l_tot);
      rowmax[static_cast<size_t>(head) * ntok + t] = m_raw;
    }
  }
  // block maxima of the raw row max and of |q_t|^2 for the max-logit refinement
  float qn2 = 0.0f;
#pragma unroll
  for (int kk = 0; kk < kD / 16; ++kk)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = static_cast<float>(qf[kk][e]);
      qn2 = fmaf(x, x, qn2);
    }
  qn2 += __shfl_xor(qn2, 32, 64);
  float v = qvalid ? m_raw : -INFINITY;
  v = wave_max(v);
  qn2 = wave_max(qvalid ? qn2 : 0.0f);
  if (lane == 0) {
    red[wave] = v;
    redq[wave] = qn2;
  }
  __syncthreads();
  if (tid == 0) {
    const float mm = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    if (mm > -INFINITY) atomic_max_float(aux + head * kAuxStride, mm);
    atomic_max_float(aux + head * kAuxStride + 1, fmaxf(fmaxf(redq[0], redq[1]), fmaxf(redq[2], redq[3])));
  }
}

// ---------------------------------------------------------------------------
// Max-logit refinement. The attention kernel's logits carry the bf16 rounding
// of K^C (relative error up to 2^-8 per element: 8 significant bits), so
// its maximum can be off by ~1e-3.
// Every logit satisfies |approx - exact| <= delta with
//   delta = (2^-8 * 1.01 + 3e-5) * max_t |q_t| * max_s |K_s|
// (bf16 rounding of K^C plus fp32 accumulation), hence the exact maximum E
// lies in [M - delta, M + delta] for the approximate maximum M, and its pair
// has an approximate logit >= M - 2 delta. The scan kernel (heads x key
// slices) re-scores the candidate rows (row max >= M - 2 delta) against their
// keys with the stored bf16 K^C and lists the candidate pairs; the exact
// kernel recomputes those pairs in fp32 from c^KV and kv_b_proj
// (K^C_s = c_s W_UK_h). Too many candidates (near-ties, e.g. q = 0) fall back
// to M, which is then within delta of E.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float refine_threshold(const float* aux, int h, int heads, float* M_out) {
  const float M = aux[h * kAuxStride];
  const float qn = sqrtf(aux[h * kAuxStride + 1]);
  const float kn = sqrtf(aux[h * kAuxStride + 2] + aux[static_cast<size_t>(heads) * kAuxStride]);
  *M_out = M;
  return M - 2.0f * (1.01f / 256.0f + 3e-5f) * qn * kn;
}

__global__ void __launch_bounds__(256) prefill_refine_scan_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ ks, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ pcu, int nseq, int heads, int64_t ntok, int64_t npad_max,
    const uint16_t* __restrict__ kc, const float* __restrict__ rowmax, const float* __restrict__ aux,
    int32_t* __restrict__ cand) {
  __shared__ int rows[kRefRows];
  __shared__ int nrows;
  __shared__ float qrow[kD];
  const int h = blockIdx.x, slice = blockIdx.y;
  const int tid = threadIdx.x;
  float M;
  const float thr = refine_threshold(aux, h, heads, &M);
  if (!(M > -INFINITY)) return;
  int32_t* c = cand + static_cast<size_t>(h) * kCandStride;
  if (tid == 0) nrows = 0;
  __syncthreads();
  for (int64_t t = tid; t < ntok; t += 256) {
    if (rowmax[static_cast<size_t>(h) * ntok + t] >= thr) {
      const int k = atomicAdd(&nrows, 1);
      if (k < kRefRows) rows[k] = static_cast<int>(t);
    }
  }
  __syncthreads();
  if (nrows > kRefRows) {
    if (tid == 0) c[1] = 1;
    return;
  }
  for (int r = 0; r < nrows; ++r) {
    const int t = rows[r];
    int lo = 0, hi = nseq - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    const int a = cu[lo];
    const int nkeys = t - a + 1;
    const int per = (nkeys + kRefSlices - 1) / kRefSlices;
    const int s0 = a + slice * per, s1 = min(t + 1, s0 + per);
    __syncthreads();
    if (tid < kD) qrow[tid] = bf16_to_f32(q[(static_cast<size_t>(t) * heads + h) * kD + tid]);
    __syncthreads();
    const uint16_t* kch = kc + (static_cast<size_t>(h) * npad_max + pcu[lo]) * kN;
    for (int s = s0 + tid; s < s1; s += 256) {
      uint4 x[kD / 8];
      const uint16_t* kr = kch + static_cast<size_t>(s - a) * kN;
      const uint16_t* sr = ks + static_cast<size_t>(s) * kS;
#pragma unroll
      for (int e = 0; e < kN / 8; ++e) x[e] = ldg16(kr + 8 * e);
#pragma unroll
      for (int e = 0; e < kS / 8; ++e) x[kN / 8 + e] = ldg16(sr + 8 * e);
      float acc = 0.0f;
#pragma unroll
      for (int e = 0; e < kD / 8; ++e) {
        const uint32_t* w4 = &x[e].x;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          acc = fmaf(qrow[8 * e + 2 * u], bf16lo(w4[u]), fmaf(qrow[8 * e + 2 * u + 1], bf16hi(w4[u]), acc));
      }
      if (acc >= thr) {
        const int k = atomicAdd(&c[0], 1);
        if (k < kRefKeys) {
          c[2 + 2 * k] = t;
          c[3 + 2 * k] = s;
        } else {
          c[1] = 1;
        }
      }
    }
  }
}

__global__ void __launch_bounds__(256) prefill_refine_exact_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ ckv, const uint16_t* __restrict__ ks,
    const uint16_t* __restrict__ w, int heads, const float* __restrict__ aux, const int32_t* __restrict__ cand,
    float scale, float* __restrict__ max_logit) {
  __shared__ float qrow[kD];
  __shared__ float crow[kR];
  __shared__ float red[8];
  const int h = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float M;
  refine_threshold(aux, h, heads, &M);
  if (!(M > -INFINITY)) return;
  const int32_t* c = cand + static_cast<size_t>(h) * kCandStride;
  const int nk = c[0];
  float best = -INFINITY;
  if (c[1] == 0 && nk <= kRefKeys) {
    for (int k = 0; k < nk; ++k) {
      const int t = c[2 + 2 * k], s = c[3 + 2 * k];
      __syncthreads();
      if (tid < kD) qrow[tid] = bf16_to_f32(q[(static_cast<size_t>(t) * heads + h) * kD + tid]);
      for (int e = tid; e < kR; e += 256) crow[e] = bf16_to_f32(ckv[static_cast<size_t>(s) * kR + e]);
      __syncthreads();
      // K^C_s[n] = sum_r c_s[r] * w[h*256 + n][r] in fp32; two threads per feature n
      const int n = tid >> 1, part = tid & 1;
      const uint16_t* wr = w + (static_cast<size_t>(h) * 256 + n) * kR + part * (kR / 2);
      uint4 x[kR / 16];
#pragma unroll
      for (int e = 0; e < kR / 16; ++e) x[e] = ldg16(wr + 8 * e);
      float kcn = 0.0f;
#pragma unroll
      for (int e = 0; e < kR / 16; ++e) {
        const uint32_t* w4 = &x[e].x;
        const float* cr = crow + part * (kR / 2) + 8 * e;
#pragma unroll
        for (int u = 0; u < 4; ++u) kcn = fmaf(cr[2 * u], bf16lo(w4[u]), fmaf(cr[2 * u + 1], bf16hi(w4[u]), kcn));
      }
      kcn += __shfl_xor(kcn, 1, 64);
      float pr = part == 0 ? qrow[n] * kcn : 0.0f;
      if (tid < kS) pr += qrow[kN + tid] * bf16_to_f32(ks[static_cast<size_t>(s) * kS + tid]);
      pr = wave_sum(pr);
      if (lane == 0) red[wave] = pr;
      __syncthreads();
      best = fmaxf(best, (red[0] + red[1]) + (red[2] + red[3]));
    }
  }
  if (tid == 0) {
    const float e = (c[1] != 0 || nk > kRefKeys || !(best > -INFINITY)) ? M : best;
    atomic_max_float(max_logit + h, e * scale);
  }
}

__global__ void prefill_aux_init_kernel(float* aux, int32_t* cand, int heads) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < (heads + 1) * kAuxStride) aux[i] = ((i % kAuxStride) == 0 && i < heads * kAuxStride) ? -INFINITY : 0.0f;
  if (i < heads) {
    cand[static_cast<size_t>(i) * kCandStride] = 0;
    cand[static_cast<size_t>(i) * kCandStride + 1] = 0;
  }
}

hipError_t launch_prefill_bf16(int heads, float scale, bool out_bf16, const void* q, const void* ckv,
                               const void* ks, const void* w_kv_b, const void* gate, const int32_t* cu,
                               int nseq, int64_t ntok, void* out, float* lse, float* max_logit, void* ws,
                               hipStream_t st) {
  const PrefillWs L = prefill_ws_layout(heads, ntok, nseq);
  char* base = static_cast<char*>(ws);
  uint16_t* kc = reinterpret_cast<uint16_t*>(base + L.kc);
  uint16_t* vt = reinterpret_cast<uint16_t*>(base + L.vt);
  int32_t* pcu = reinterpret_cast<int32_t*>(base + L.pcu);
  int32_t* order = reinterpret_cast<int32_t*>(base + L.order);
  int32_t* toff = reinterpret_cast<int32_t*>(base + L.toff);
  int32_t* hdr = reinterpret_cast<int32_t*>(base + L.hdr);
  float* rowmax = reinterpret_cast<float*>(base + L.rowmax);
  float* aux = reinterpret_cast<float*>(base + L.aux);
  int32_t* cand = reinterpret_cast<int32_t*>(base + L.cand);

  {
    TimedScope ts_("prefill_aux_init", st);
    hipLaunchKernelGGL(prefill_aux_init_kernel, dim3((heads + 1) * kAuxStride / 256 + 1), dim3(256), 0, st, aux,
                       cand, heads);
  }
  {
    TimedScope ts_("prefill_plan", st);
    hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(256), 0, st, cu, nseq, pcu, order, toff, hdr);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const dim3 eg(2 * heads, static_cast<unsigned>(L.npad_max / kExBM));
  {
    TimedScope ts_("prefill_expand", st);
    hipLaunchKernelGGL(prefill_expand_kernel, eg, dim3(256), 0, st, static_cast<const uint16_t*>(ckv),
                       static_cast<const uint16_t*>(w_kv_b), cu, nseq, pcu, hdr, L.npad_max,
                       static_cast<const uint16_t*>(ks), kc, vt, aux);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  // upper bound on query tiles: sum over sequences of ceil(L/128) <= ntok/128 + nseq
  const int64_t tiles_max = (ntok + kPrefBM - 1) / kPrefBM + nseq;
  const int64_t total_max = tiles_max * heads;
  const int64_t grid = ((total_max + 7) / 8) * 8;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (out_bf16) {
    {
      TimedScope ts_("prefill_attn", st);
      hipLaunchKernelGGL(prefill_attn_kernel<true>, dim3(static_cast<unsigned>(grid)), dim3(256), 0, st,
                         static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(ks),
                         static_cast<const uint16_t*>(gate), cu, pcu, order, toff, hdr, nseq, heads, ntok,
                         L.npad_max, kc, vt, scale, out, lse, rowmax, aux);
    }
  } else {
    {
      TimedScope ts_("prefill_attn", st);
      hipLaunchKernelGGL(prefill_attn_kernel<false>, dim3(static_cast<unsigned>(grid)), dim3(256), 0, st,
                         static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(ks),
                         static_cast<const uint16_t*>(gate), cu, pcu, order, toff, hdr, nseq, heads, ntok,
                         L.npad_max, kc, vt, scale, out, lse, rowmax, aux);
    }
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    TimedScope ts_("prefill_refine_scan", st);
    hipLaunchKernelGGL(prefill_refine_scan_kernel, dim3(heads, kRefSlices), dim3(256), 0, st,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(ks), cu, pcu, nseq, heads, ntok,
                       L.npad_max, kc, rowmax, aux, cand);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    TimedScope ts_("prefill_refine_exact", st);
    hipLaunchKernelGGL(prefill_refine_exact_kernel, dim3(heads), dim3(256), 0, st, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(ckv), static_cast<const uint16_t*>(ks),
                       static_cast<const uint16_t*>(w_kv_b), heads, aux, cand, scale, max_logit);
  }
  return hipGetLastError();
}

}  // namespace mla
