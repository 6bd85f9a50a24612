// Training-form gated MLA prefill, bf16 inputs, Kimi K3 head shape
// (R = 512, S = 64, N = 128, V = 128), gfx950 MFMA.
//
// Follows the equation list of "Kimi K3 · Gated MLA · OpenModelAtlas":
//   [k^C v] = c^KV W_UKV (expansion, materialised once into the workspace),
//   K_h = [K^C_h, k^S], S = Q K^T / sqrt(192), causal softmax, O~ = A V,
//   o = sigma(g) . reshape(O~); plus the per-head maximum of S that QK-Clip
//   ("SOTA-131") needs.
//
// Five launches: a one-workgroup plan (per-sequence padded offsets, a
// longest-first tile order, and the clearing of the max-logit state), the
// expansion GEMM, the attention kernel, and the two max-logit refinement
// kernels.
#include <algorithm>
#include <type_traits>

#include "mla_common.h"
#include "mla_internal.h"
#include "timing.h"

namespace mla {

// ---------------------------------------------------------------------------
// Plan: pcu[s] = start of sequence s in the padded workspace (each sequence
// rounded up to 64 rows), order[] = sequences by descending length (ties by
// index), toff[r] = first query tile of the r-th sequence in that order,
// hdr = {tiles, padded rows}. The same single workgroup also clears the
// max-logit refinement state and, unless the caller accumulates, sets the
// max-logit slots to -inf.
//
// Up to 64 sequences: one wave, one sequence per lane; the prefixes are wave
// shuffle scans and the order a rank count over the lanes. Otherwise:
// lengths are read once per chunk of kPlanSortMax sequences into LDS; both
// prefixes are block scans over a chunk (16 consecutive values per thread,
// wave shuffles, one LDS exchange of the four wave totals). Up to
// kPlanSortMax sequences are ordered by a bitonic sort of 64-bit keys in LDS
// (high word = length mapped so that ascending keys mean descending lengths,
// low word = index); past that the sequences keep their index order.
// ---------------------------------------------------------------------------
constexpr int kPlanThreads = 256;
constexpr int kPlanWaves = kPlanThreads / 64;
constexpr int kPlanSortMax = 4096;
constexpr int kPlanPer = kPlanSortMax / kPlanThreads;
constexpr int kPlanPairs = kPlanSortMax / 2 / kPlanThreads;

// Exclusive scan of val(0 .. n-1), n <= kPlanSortMax, offset by carry; calls
// out(i, prefix_i) and returns carry + the sum. All threads must call it.
template <class Val, class Out>
__device__ __forceinline__ int plan_scan(int n, int carry, int* s_wave, Val val, Out out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, b = tid * kPlanPer;
  int v[kPlanPer];
  int sum = 0;
#pragma unroll
  for (int j = 0; j < kPlanPer; ++j) {
    v[j] = b + j < n ? val(b + j) : 0;
    sum += v[j];
  }
  int x = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  int run = carry + x - sum, total = 0;
#pragma unroll
  for (int w = 0; w < kPlanWaves; ++w) {
    const int t = s_wave[w];
    run += w < wave ? t : 0;
    total += t;
  }
#pragma unroll
  for (int j = 0; j < kPlanPer; ++j) {
    if (b + j < n) out(b + j, run);
    run += v[j];
  }
  __syncthreads();
  return carry + total;
}

__global__ void __launch_bounds__(kPlanThreads) prefill_plan_kernel(const int32_t* __restrict__ cu, int nseq,
                                                                    int32_t* __restrict__ pcu,
                                                                    int32_t* __restrict__ order,
                                                                    int32_t* __restrict__ toff,
                                                                    int32_t* __restrict__ hdr, int heads,
                                                                    float* __restrict__ aux,
                                                                    int32_t* __restrict__ cand,
                                                                    float* __restrict__ ml_init) {
  __shared__ uint64_t s_key[kPlanSortMax];
  __shared__ int s_len[kPlanSortMax];
  __shared__ int s_wave[kPlanWaves];
  const int tid = threadIdx.x;
  for (int i = tid; i < (heads + 1) * kAuxStride; i += kPlanThreads)
    aux[i] = ((i % kAuxStride) == 0 && i < heads * kAuxStride) ? -INFINITY : 0.0f;
  for (int i = tid; i < kCandHeadCount + heads; i += kPlanThreads) cand[i] = 0;
  if (ml_init)
    for (int i = tid; i < heads; i += kPlanThreads) ml_init[i] = -INFINITY;
  auto pad_rows = [](int L) { return (L + kSeqPad - 1) / kSeqPad * kSeqPad; };
  auto q_tiles = [](int L) { return (L + kPrefBM - 1) / kPrefBM; };

  if (nseq <= 64) {
    // One wave, one sequence per lane, everything in registers.
    if (tid < 64) {
      const int lane = tid;
      const int L = lane < nseq ? cu[lane + 1] - cu[lane] : 0;
      auto incl_scan = [&](int x) {
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int y = __shfl_up(x, off, 64);
          if (lane >= off) x += y;
        }
        return x;
      };
      const int a = lane < nseq ? pad_rows(L) : 0, pa = incl_scan(a);
      if (lane < nseq) pcu[lane] = pa - a;
      int rank = 0;
      for (int s = 0; s < nseq; ++s) {
        const int Ls = __builtin_amdgcn_readlane(L, s);
        rank += (Ls > L) || (Ls == L && s < lane);
      }
      int at = 0;  // the sequence ranked lane-th
      for (int s = 0; s < nseq; ++s) at = __builtin_amdgcn_readlane(rank, s) == lane ? s : at;
      const int b = lane < nseq ? q_tiles(__shfl(L, at, 64)) : 0, pb = incl_scan(b);
      if (lane < nseq) {
        order[lane] = at;
        toff[lane] = pb - b;
      }
      if (lane == 63) {
        pcu[nseq] = pa;
        toff[nseq] = pb;
        hdr[0] = pb;
        hdr[1] = pa;
      }
    }
    return;
  }

  const bool sort = nseq <= kPlanSortMax;
  int p = 0, t = 0;
  for (int c0 = 0; c0 < nseq; c0 += kPlanSortMax) {
    const int n = min(kPlanSortMax, nseq - c0);
    for (int i = tid; i < n; i += kPlanThreads) s_len[i] = cu[c0 + i + 1] - cu[c0 + i];
    __syncthreads();
    p = plan_scan(n, p, s_wave, [&](int i) { return pad_rows(s_len[i]); },
                  [&](int i, int x) { pcu[c0 + i] = x; });
    if (!sort)
      t = plan_scan(n, t, s_wave, [&](int i) { return q_tiles(s_len[i]); },
                    [&](int i, int x) {
                      order[c0 + i] = c0 + i;
                      toff[c0 + i] = x;
                    });
  }
  if (sort) {
    // s_len holds all nseq lengths (one chunk).
    int n2 = 1;
    while (n2 < nseq) n2 <<= 1;
    for (int i = tid; i < n2; i += kPlanThreads) {
      uint64_t key = ~uint64_t{0};
      if (i < nseq) {
        const uint32_t hi = 0xffffffffu - (static_cast<uint32_t>(s_len[i]) ^ 0x80000000u);
        key = (static_cast<uint64_t>(hi) << 32) | static_cast<uint32_t>(i);
      }
      s_key[i] = key;
    }
    __syncthreads();
    // Each step: pair q = tid + 256 m takes keys i (bit j clear) and i + j;
    // all of a thread's loads are issued before its compare-and-swaps.
    for (int k = 2, lk = 1; k <= n2; k <<= 1, ++lk)
      for (int j = k >> 1, lj = lk - 1; j > 0; j >>= 1, --lj) {
        uint64_t a[kPlanPairs], c[kPlanPairs];
#pragma unroll
        for (int m = 0; m < kPlanPairs; ++m) {
          const int q = tid + m * kPlanThreads, i = ((q >> lj) << (lj + 1)) | (q & (j - 1));
          if (q < n2 / 2) {
            a[m] = s_key[i];
            c[m] = s_key[i + j];
          }
        }
#pragma unroll
        for (int m = 0; m < kPlanPairs; ++m) {
          const int q = tid + m * kPlanThreads, i = ((q >> lj) << (lj + 1)) | (q & (j - 1));
          if (q < n2 / 2 && (a[m] > c[m]) == ((i & k) == 0)) {
            s_key[i] = c[m];
            s_key[i + j] = a[m];
          }
        }
        __syncthreads();
      }
    auto seq_at = [&](int r) { return static_cast<int>(static_cast<uint32_t>(s_key[r])); };
    t = plan_scan(nseq, 0, s_wave, [&](int r) { return q_tiles(s_len[seq_at(r)]); },
                  [&](int r, int x) {
                    order[r] = seq_at(r);
                    toff[r] = x;
                  });
  }
  if (tid == 0) {
    pcu[nseq] = p;
    toff[nseq] = t;
    hdr[0] = t;
    hdr[1] = p;
  }
}

// ---------------------------------------------------------------------------
// Expansion: [K^C_h | V_h][p] = c^KV[src(p)] W_UKV[:, 256h : 256h+256] over
// padded rows p. One workgroup = 256 padded rows (four key tiles) x the 256
// columns of one head; 8 waves, wave w owns rows 64 (w & 3) .. +63 of the
// K^C half (w < 4) or of the V half. K = 512 in 8 steps of 64: both operand
// tiles of a step (256 rows x 128 bytes each) are copied straight into LDS
// (buffer loads to LDS, no register staging) one step ahead, into two slots.
//
// Each copy instruction moves 8 whole 128-byte row segments (eight lanes per
// row), so every request is a full cache line. LDS tile layout (one operand,
// 256 rows x eight 16-byte k-units): unit (r, c) at 64 (r / 8) + 8 (r % 8) +
// (c ^ ((r / 2) % 8)); a 16-lane group of a fragment read (16 consecutive
// rows, one k-unit) then falls into 16 different bank groups.
//
// Both halves are stored straight from the accumulators with 16-byte stores:
// V is formed as C = c^KV W_V (accumulator lane = feature d, its rows = keys)
// and lands in V^T units of eight keys in value-operand order (vperm16); K^C
// is formed transposed, C^T = W_K c^KV^T (lane = key, rows = features), and
// lands in units of eight features in that same order: unit u of a K^C row
// holds features kperm(8u .. 8u+7), kperm(n) = (n & ~15) | vperm16(n & 15).
// The attention kernel loads q^C in that feature order. The head-0 workgroups
// also write the padded k^S copy.
// ---------------------------------------------------------------------------
constexpr int kExRows = 256;      // padded rows per workgroup
constexpr int kExThreads = 512;
constexpr int kExSteps = kR / 64;  // k-steps of 64
constexpr int kExUnits = kExRows * 8;  // 16-byte units per operand slot
constexpr int kExGroupRows = 4, kExGroupHeads = 8, kExGroup = kExGroupRows * kExGroupHeads;

__global__ void __launch_bounds__(kExThreads) prefill_expand_kernel(
    const uint16_t* __restrict__ ckv, const uint16_t* __restrict__ w, const int32_t* __restrict__ cu,
    int nseq, const int32_t* __restrict__ pcu, const int32_t* __restrict__ hdr, int64_t npad_max, int64_t ntok,
    int heads, const uint16_t* __restrict__ ks, uint16_t* __restrict__ kc, uint16_t* __restrict__ vt,
    uint16_t* __restrict__ ksp, float* __restrict__ aux) {
  __shared__ uint4 Cs0[kExUnits], Cs1[kExUnits];   // c^KV slots
  __shared__ uint4 Ws0[kExUnits], Ws1[kExUnits];   // W_UKV slots
  __shared__ int src_row[kExRows];
  __shared__ float red[8];

  // ---- work item: groups of kExGroupRows row tiles x kExGroupHeads heads,
  // consecutive groups on the same XCD ----
  // the row tiles of the padded tokens of this call (hdr[1]), not of the
  // workspace's bound npad_max: the items are dealt to the XCDs in equal
  // contiguous ranges, and counting empty tiles would leave the last XCDs
  // nearly idle
  const int npad = hdr[1];
  const int nrt = (npad + kExRows - 1) / kExRows;
  const int nrg = (nrt + kExGroupRows - 1) / kExGroupRows, nhg = (heads + kExGroupHeads - 1) / kExGroupHeads;
  const int per_xcd = (nrg * nhg * kExGroup + 7) >> 3;
  const int slot = blockIdx.x >> 3;
  if (slot >= per_xcd) return;
  const int item = (blockIdx.x & 7) * per_xcd + slot;
  const int grp = item / kExGroup, gi = item - grp * kExGroup;
  if (grp >= nrg * nhg) return;
  const int rg = grp / nhg, hg = grp - rg * nhg;
  const int rt = rg * kExGroupRows + gi % kExGroupRows;
  const int head = hg * kExGroupHeads + gi / kExGroupRows;
  if (rt >= nrt || head >= heads) return;
  const int m0 = rt * kExRows;
  if (m0 >= npad) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar branches)
  const int g = lane >> 5, l32 = lane & 31;
  const int wm = wave & 3, half = wave >> 2;

  if (tid < kExRows) {
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

  // ---- staging: copy q of wave w covers rows 8 (4 w + q) .. +7; lane i
  // takes row 8 (4 w + q) + i / 8 and k-unit (i % 8) ^ ((row / 2) % 8). The
  // c^KV resource starts at the tile's first source row (its rows are
  // consecutive source rows, with padding between sequences), so 32-bit
  // offsets suffice; padding rows read past its end and get zeros.
  int src0 = 0x7fffffff;
#pragma unroll
  for (int j = 0; j < kExRows / 64; ++j) {
    const int v = src_row[64 * j + lane];
    if (v >= 0) src0 = min(src0, v);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) src0 = min(src0, __shfl_xor(src0, o));
  if (src0 == 0x7fffffff) src0 = 0;
  src0 = __builtin_amdgcn_readfirstlane(src0);   // uniform after the reduction
  const auto rs_c = make_rsrc(ckv + static_cast<size_t>(src0) * kR, kExRows * kR * 2);
  const auto rs_w = make_rsrc(w + static_cast<size_t>(head) * 256 * kR, 256 * kR * 2);
  uint32_t voff_c[4], voff_w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 8 * (4 * wave + q) + (lane >> 3), c = (lane & 7) ^ ((r >> 1) & 7);
    const int src = src_row[r];
    voff_c[q] = src >= 0 ? static_cast<uint32_t>(src - src0) * (kR * 2) + 16 * c : 0x80000000u;   // padding rows: zeros
    voff_w[q] = static_cast<uint32_t>(r) * (kR * 2) + 16 * c;
  }
  auto issue = [&](uint4* cd, uint4* wd, int st) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      dma16_buf(rs_c, voff_c[q], 128 * st, cd + 64 * (4 * wave + q));
      dma16_buf(rs_w, voff_w[q], 128 * st, wd + 64 * (4 * wave + q));
    }
  };
  auto frag = [&](const uint4* t, int r0, int kh) {   // rows r0 .. r0+31, k-units 2 kh + g
    const int r = r0 + l32, c = 2 * kh + g;
    return as_bf16x8(t[64 * (r >> 3) + 8 * (r & 7) + (c ^ ((r >> 1) & 7))]);
  };

  // acc: K half (transposed C^T): acc[2 fb + kb], fb = feature block (4), kb = key block (2);
  //      V half: acc[4 kb + fb]. Each half runs its own copy of the loop (no
  //      register joins between the two operand orders).
  const size_t tiles_h = static_cast<size_t>(head) * (npad_max / kPrefBN);
  float n2 = 0.0f;   // |K^C_key|^2 of this lane's keys (bf16 values), K half only
  auto run = [&](auto HALF) {
    constexpr int H = decltype(HALF)::value;
    f32x16 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = f32x16{};

    auto step = [&](const uint4* cs, const uint4* ws) {
#pragma unroll
      for (int kh = 0; kh < 4; ++kh) {
        bf16x8 cf[2], wf[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) cf[kb] = frag(cs, 64 * wm + 32 * kb, kh);
#pragma unroll
        for (int fb = 0; fb < 4; ++fb) wf[fb] = frag(ws, 128 * H + 32 * fb, kh);
        if constexpr (H == 0) {
#pragma unroll
          for (int fb = 0; fb < 4; ++fb)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) acc[2 * fb + kb] = mfma32(wf[fb], cf[kb], acc[2 * fb + kb]);
        } else {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int fb = 0; fb < 4; ++fb) acc[4 * kb + fb] = mfma32(cf[kb], wf[fb], acc[4 * kb + fb]);
        }
      }
    };
    issue(Cs0, Ws0, 0);
    wait_vmcnt<0>();
    __syncthreads();
    for (int st = 0; st < kExSteps; st += 2) {
      issue(Cs1, Ws1, st + 1);   // slot 1 was last read by step st - 1
      __builtin_amdgcn_sched_barrier(0);
      step(Cs0, Ws0);
      wait_vmcnt<0>();
      __syncthreads();
      if (st + 2 < kExSteps) issue(Cs0, Ws0, st + 2);
      __builtin_amdgcn_sched_barrier(0);
      step(Cs1, Ws1);
      wait_vmcnt<0>();
      __syncthreads();
    }

    // ---- store: 16-byte units straight from the accumulators ----
    if constexpr (H == 0) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int p = m0 + 64 * wm + 32 * kb + l32;          // this lane's key (padded row)
        uint16_t* dst = kc + (tiles_h + p / kPrefBN) * kTileElems + (p % kPrefBN) * 8;
        float s2 = 0.0f;
#pragma unroll
        for (int fb = 0; fb < 4; ++fb)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const f32x16& a = acc[2 * fb + kb];
            uint32_t wv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              wv[e] = pack_bf16x2(a[8 * hh + 2 * e], a[8 * hh + 2 * e + 1]);
              s2 = fmaf(bf16lo(wv[e]), bf16lo(wv[e]), fmaf(bf16hi(wv[e]), bf16hi(wv[e]), s2));
            }
            const int u = 4 * fb + 2 * hh + g;                  // features kperm(8u .. 8u+7)
            stg16(dst + u * (kPrefBN * 8), make_uint4(wv[0], wv[1], wv[2], wv[3]));
          }
        n2 = fmaxf(n2, xor32_sum(s2));
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int fb = 0; fb < 4; ++fb)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const f32x16& a = acc[4 * kb + fb];
            const int p0 = m0 + 64 * wm + 32 * kb + 16 * hh;    // first key of the 16-key group
            const int d = 32 * fb + l32;
            const int u = ((p0 % kPrefBN) >> 3) + g;            // keys at value-operand positions 8u .. 8u+7
            uint16_t* dst = vt + (tiles_h + p0 / kPrefBN) * kTileElems + (u * kV + d) * 8;
            stg16(dst, make_uint4(pack_bf16x2(a[8 * hh], a[8 * hh + 1]), pack_bf16x2(a[8 * hh + 2], a[8 * hh + 3]),
                                  pack_bf16x2(a[8 * hh + 4], a[8 * hh + 5]), pack_bf16x2(a[8 * hh + 6], a[8 * hh + 7])));
          }
    }
  };
  if (half == 0) run(std::integral_constant<int, 0>{});
  else run(std::integral_constant<int, 1>{});
  // largest squared norm of a stored K^C row (and, once, of a k^S row): the
  // error bound of the max-logit refinement
  n2 = wave_max(n2);
  if (lane == 0) red[wave] = n2;
  if (head == 0) {
    // padded k^S copy (tile-blocked, zero rows past each sequence) and the largest |k^S_s|^2
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int id = tid + kExThreads * c;   // 256 rows x 8 units
      const int r = id & 63, u = (id >> 6) & 7, tl = id >> 9;
      const int src = src_row[tl * kPrefBN + r];
      const uint4 v = src >= 0 ? ldg16(ks + static_cast<size_t>(src) * kS + 8 * u) : make_uint4(0, 0, 0, 0);
      stg16(ksp + (static_cast<size_t>(m0 / kPrefBN + tl) * (kS / 8) + u) * (kPrefBN * 8) + r * 8, v);
    }
    float s2 = 0.0f;
    if (tid < kExRows && src_row[tid] >= 0) {
#pragma unroll
      for (int u = 0; u < kS / 8; ++u) {
        const uint4 v = ldg16(ks + static_cast<size_t>(src_row[tid]) * kS + 8 * u);
        const uint32_t* x = &v.x;
#pragma unroll
        for (int e = 0; e < 4; ++e) s2 = fmaf(bf16lo(x[e]), bf16lo(x[e]), fmaf(bf16hi(x[e]), bf16hi(x[e]), s2));
      }
    }
    s2 = wave_max(s2);
    if (lane == 0 && wave < kExRows / 64) atomic_max_float(aux + static_cast<size_t>(heads) * kAuxStride, s2);
  }
  __syncthreads();
  if (tid == 0) {
    float mm = red[0];
    for (int i = 1; i < 4; ++i) mm = fmaxf(mm, red[i]);
    atomic_max_float(aux + head * kAuxStride + 2, mm);
  }
}

// ---------------------------------------------------------------------------
// QK-norm variant ("SOTA-131", Variations and Mechanism): each head's query is
// divided by the root mean square of its D = 192 features and multiplied by a
// per-feature weight, then rounded to bf16 (the attention's operand). The
// attention kernel and the max-logit refinement both form it, with the same
// arithmetic in the same order, so they use bit-identical queries: the sum of
// squares is two fp32 fma chains, one per lane half of the attention's query
// layout (half g holds features 16 kk + 4 g .. +3 and 16 kk + 8 + 4 g .. +3 for
// kk < 8, then 16 kk + 8 g .. +7 for kk = 8 .. 11), added at the end.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int qslot_feature(int g, int kk, int e) {
  return kk < kN / 16 ? 16 * kk + 8 * (e >> 2) + 4 * g + (e & 3) : 16 * kk + 8 * g + e;
}
__device__ __forceinline__ float qnorm_scale(float sumsq, float eps) {
  return 1.0f / sqrtf(sumsq / static_cast<float>(kD) + eps);
}
__device__ __forceinline__ float qnorm_value(float x, float r, const uint16_t* w, int f) {
  return bf16_to_f32(f32_to_bf16(x * r * (w ? bf16_to_f32(w[f]) : 1.0f)));
}
// Sum of squares of one bf16 query row in the attention kernel's order.
__device__ __forceinline__ float qnorm_sumsq_row(const uint16_t* qrow) {
  float half[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    float ss = 0.0f;
#pragma unroll
    for (int kk = 0; kk < kD / 16; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = bf16_to_f32(qrow[qslot_feature(g, kk, e)]);
        ss = fmaf(x, x, ss);
      }
    half[g] = ss;
  }
  return half[0] + half[1];
}

// ---------------------------------------------------------------------------
// Attention. One workgroup = one head x 128 queries of one sequence; 4 waves
// of 32 queries, two workgroups per CU (80 KB of LDS and at most 256 VGPRs
// each), so that one workgroup's prologue (query and first tile loads) and
// epilogue (output stores) overlap the other's tile loop. Scores are formed
// transposed (S^T = K Q^T) so
// that each lane owns one query column: the row max/sum and the output
// rescale stay in the lane. Keys are visited in tiles of 64 up to the
// diagonal (tiles above it are skipped); a wave's last tile is its only
// masked one.
//
// K tiles ([24 units][64 keys]: K^C units then k^S units) and V^T tiles
// ([8 units][128 d]) live in two double-buffered LDS rings, copied straight
// from the tile-blocked workspace (no register staging) one tile ahead; a
// wave's 16-lane group reads 16 consecutive 16-byte units (no bank
// conflicts). Software pipeline per wave and tile j:
//   [B] S(j+1) = K(j+1) Q^T on the matrix cores while the VALU turns S(j)
//       into bf16 probabilities;
//   [C] O^T += V(j)^T P(j)^T on the matrix cores while the VALU masks and
//       takes the row max of S(j+1).
// The softmax keeps a per-query reference max that moves only when a tile's
// max exceeds it by more than 2^8 (in exp2 units), so the output rescale is
// rare; probabilities stay <= 2^8, exact in fp32 and bf16 range.
// ---------------------------------------------------------------------------
constexpr int kAttnWaves = kPrefBM / 32;                 // one wave per 32 queries
constexpr int kAttnThreads = 64 * kAttnWaves;
constexpr int kKUnits = kD / 8;                          // 16-byte units per key row (24)
constexpr int kKTile = kPrefBN * kKUnits;                // 1536 units = 24 KB
constexpr int kVTile = kV * (kPrefBN / 8);               // 1024 units = 16 KB
constexpr int kKcCopies = (kN / 8) / kAttnWaves;         // 1 KB copies per wave per tile: K^C,
constexpr int kKsCopies = (kS / 8) / kAttnWaves;         //   k^S
constexpr int kVtCopies = (kVTile / 64) / kAttnWaves;    //   and V^T
static_assert(kKcCopies * kAttnWaves == kN / 8 && kKsCopies * kAttnWaves == kS / 8 &&
                  kVtCopies * kAttnWaves == kVTile / 64, "tile copies split evenly over the waves");
constexpr float kRescaleLog2 = 8.0f;

// Issue order of the overlapped tile body. qk: score MFMA idx = 12 blk + kk
// (else value MFMA idx = 4 jj + db); pair: probability pair formed with it;
// mx: group of four elements of score block 0 folded into the row max.
struct Ovl {
  bool qk;
  int8_t idx, pair, mx;
};
constexpr Ovl kOvl[] = {
    {true, 0, 0, -1},   {true, 1, 1, -1},   {true, 2, 2, -1},   {true, 3, 3, -1},   {true, 4, -1, -1},
    {true, 5, -1, -1},  {true, 6, 4, -1},   {false, 0, -1, -1}, {true, 7, 5, -1},   {false, 1, -1, -1},
    {true, 8, 6, -1},   {false, 2, -1, -1}, {true, 9, 7, -1},   {false, 3, -1, -1}, {true, 10, 8, -1},
    {false, 4, -1, -1}, {true, 11, 9, -1},  {false, 5, -1, -1}, {true, 12, 10, -1}, {false, 6, -1, -1},
    {true, 13, 11, -1}, {false, 7, -1, -1}, {true, 14, 12, -1}, {false, 8, -1, 0},  {true, 15, 13, -1},
    {false, 9, -1, 1},  {true, 16, 14, -1}, {false, 10, -1, 2}, {true, 17, 15, -1}, {false, 11, -1, 3},
    {true, 18, -1, -1}, {false, 12, -1, -1}, {true, 19, -1, -1}, {false, 13, -1, -1}, {true, 20, -1, -1},
    {false, 14, -1, -1}, {true, 21, -1, -1}, {false, 15, -1, -1}, {true, 22, -1, -1}, {true, 23, -1, -1},
};
constexpr int kOvlLen = sizeof(kOvl) / sizeof(kOvl[0]);
constexpr int kRing = 4;   // LDS operand fragments in flight
static_assert(kOvlLen == 40, "24 score + 16 value MFMAs");

template <bool OUT_BF16>
__global__ void __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) prefill_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ ksp, const uint16_t* __restrict__ gate,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ pcu, const int32_t* __restrict__ order,
    const int32_t* __restrict__ toff, const int32_t* __restrict__ hdr, int nseq, int heads,
    int64_t ntok, int64_t npad_max, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vt,
    float scale, void* __restrict__ out, float* __restrict__ lse, float* __restrict__ rowmax,
    float* __restrict__ aux, int qnorm, const uint16_t* __restrict__ qn_w, float qn_eps, int hgroup) {
  __shared__ uint4 K0[kKTile];
  __shared__ uint4 K1[kKTile];
  __shared__ uint4 V0[kVTile];
  __shared__ uint4 V1[kVTile];

  // ---- work item. Blocks are dealt to the 8 XCDs in turn. With 8 heads or
  // more, XCD x owns the heads [x H / 8, (x + 1) H / 8) (so a head's K and V
  // stay in one L2) and takes them hgroup at a time, the group's query tiles
  // interleaved in the tile order (longest first): the heaviest tiles of
  // every group start early, which evens out the end of the launch, while
  // only hgroup heads' K and V are being read at a time. With fewer heads the
  // (head, tile) items are split evenly over the XCDs. ----
  const int ntiles = hdr[0];
  const int b = blockIdx.x;
  const int x = b & 7, slot = b >> 3;
  int head, tile;
  if (heads >= 8) {
    const int h0 = x * heads / 8, nh = (x + 1) * heads / 8 - h0;
    if (slot >= nh * ntiles) return;
    const int grp = slot / (hgroup * ntiles), rem = slot - grp * hgroup * ntiles;
    const int ng = min(hgroup, nh - hgroup * grp);
    tile = rem / ng;
    head = h0 + hgroup * grp + (rem - tile * ng);
  } else {
    const int total = ntiles * heads, per_xcd = (total + 7) >> 3;
    const int item = x * per_xcd + slot;
    if (slot >= per_xcd || item >= total) return;
    head = item / ntiles;
    tile = item - head * ntiles;
  }
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
  const int qw = q0 + 32 * wave;                 // first query of this wave
  const int qi = qw + l32;                       // this lane's query (sequence-local)
  const bool qvalid = qi < L;
  const int nkv = min(L, q0 + kPrefBM);
  const int nkt = (nkv + kPrefBN - 1) / kPrefBN;                     // tiles staged by the workgroup
  const int nkt_w = qw < L ? min(nkt, (qw + 31) / kPrefBN + 1) : 0;  // tiles this wave uses

  // ---- queries, held as MFMA B operands for the whole loop; the q^C
  // features in the stored K^C order kperm (two 8-byte halves per fragment) ----
  bf16x8 qf[kD / 16];
  {
    const uint16_t* qrow = q + (static_cast<size_t>(a0 + (qvalid ? qi : 0)) * heads + head) * kD;
#pragma unroll
    for (int kk = 0; kk < kN / 16; ++kk) {
      uint2 lo = make_uint2(0, 0), hi = make_uint2(0, 0);
      if (qvalid) {
        lo = *reinterpret_cast<const uint2*>(qrow + 16 * kk + 4 * g);
        hi = *reinterpret_cast<const uint2*>(qrow + 16 * kk + 8 + 4 * g);
      }
      qf[kk] = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
    }
#pragma unroll
    for (int kk = kN / 16; kk < kD / 16; ++kk)
      qf[kk] = as_bf16x8(qvalid ? ldg16(qrow + 16 * kk + 8 * g) : make_uint4(0, 0, 0, 0));
  }
  if (qnorm) {
    // QK-norm: this lane half's fma chain, the other half's added, then
    // x r w rounded to bf16 (invalid lanes keep zeros)
    float ss = 0.0f;
#pragma unroll
    for (int kk = 0; kk < kD / 16; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = static_cast<float>(qf[kk][e]);
        ss = fmaf(x, x, ss);
      }
    const float r = qvalid ? qnorm_scale(ss + __shfl_xor(ss, 32, 64), qn_eps) : 0.0f;
#pragma unroll
    for (int kk = 0; kk < kD / 16; ++kk) {
      bf16x8 v = qf[kk];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        v[e] = static_cast<__bf16>(qnorm_value(static_cast<float>(qf[kk][e]), r, qn_w, qslot_feature(g, kk, e)));
      qf[kk] = v;
    }
  }

  // tile-blocked operands of this head and sequence (tile index = padded row / 64)
  const size_t tb = static_cast<size_t>(pbase / kPrefBN);
  const uint16_t* kc_h = kc + (static_cast<size_t>(head) * (npad_max / kPrefBN) + tb) * kTileElems;
  const uint16_t* vt_h = vt + (static_cast<size_t>(head) * (npad_max / kPrefBN) + tb) * kTileElems;
  const uint16_t* ks_t = ksp + tb * (kPrefBN * kS);

  // ---- tile copies: 1 KB blocks, lane i's 16 bytes at block + 16 i. Buffer
  // loads (not flat/global ones) keep the compiler's LDS-read waits partial.
  const uint32_t seq_tiles = static_cast<uint32_t>((L + kPrefBN - 1) / kPrefBN);
  const auto rs_kc = make_rsrc(kc_h, seq_tiles * kTileElems * 2);
  const auto rs_vt = make_rsrc(vt_h, seq_tiles * kTileElems * 2);
  const auto rs_ks = make_rsrc(ks_t, seq_tiles * kPrefBN * kS * 2);
  const uint32_t lane16 = 16u * lane;
  auto dma_k = [&](uint4* dst, int j) {
    const uint32_t so = static_cast<uint32_t>(j) * (kTileElems * 2);
#pragma unroll
    for (int c = 0; c < kKcCopies; ++c) {
      const int blk = kKcCopies * wave + c;
      dma16_buf(rs_kc, lane16 + blk * 1024, so, dst + blk * 64);
    }
    const uint32_t sos = static_cast<uint32_t>(j) * (kPrefBN * kS * 2);
#pragma unroll
    for (int c = 0; c < kKsCopies; ++c) {
      const int blk = kKsCopies * wave + c;
      dma16_buf(rs_ks, lane16 + blk * 1024, sos, dst + (kN / 8 + blk) * 64);
    }
  };
  auto dma_v = [&](uint4* dst, int j) {
    const uint32_t so = static_cast<uint32_t>(j) * (kTileElems * 2);
#pragma unroll
    for (int c = 0; c < kVtCopies; ++c) {
      const int blk = kVtCopies * wave + c;
      dma16_buf(rs_vt, lane16 + blk * 1024, so, dst + blk * 64);
    }
  };

  // copy c of this wave's share of a step: K^C blocks, then k^S blocks (tile
  // jk into kdst), then V^T blocks (tile jv into vdst)
  constexpr int kStepCopies = kKcCopies + kKsCopies + kVtCopies;
  auto dma_one = [&](int c, uint4* kdst, int jk, uint4* vdst, int jv) {
    // (the block offset goes into the scalar offset: one address VGPR for all copies)
    const int w = __builtin_amdgcn_readfirstlane(wave);
    if (c < kKcCopies) {
      const int blk = kKcCopies * w + c;
      dma16_buf(rs_kc, lane16, static_cast<uint32_t>(jk) * (kTileElems * 2) + blk * 1024, kdst + blk * 64);
    } else if (c < kKcCopies + kKsCopies) {
      const int blk = kKsCopies * w + (c - kKcCopies);
      dma16_buf(rs_ks, lane16, static_cast<uint32_t>(jk) * (kPrefBN * kS * 2) + blk * 1024, kdst + (kN / 8 + blk) * 64);
    } else {
      const int blk = kVtCopies * w + (c - kKcCopies - kKsCopies);
      dma16_buf(rs_vt, lane16, static_cast<uint32_t>(jv) * (kTileElems * 2) + blk * 1024, vdst + blk * 64);
    }
  };

  // LDS operand addresses: K unit (2kk + g) * 64 + 32 blk + l32, V^T unit
  // (2jj + g) * 128 + 32 db + l32 (a 16-lane group reads 16 consecutive units)
  auto kfrag = [&](const uint4* kt, int f) {   // f = 2 kk + blk
    return as_bf16x8(kt[(2 * (f >> 1) + g) * kPrefBN + 32 * (f & 1) + l32]);
  };
  auto vfrag = [&](const uint4* vtile, int f) {   // f = 4 jj + db
    return as_bf16x8(vtile[(2 * (f >> 2) + g) * kV + 32 * (f & 3) + l32]);
  };
  constexpr int kQkMfma = 2 * (kD / 16);   // 24
  constexpr int kPvMfma = 4 * (kV / 32);   // 16
  constexpr int kPfK = 4, kPfV = 4;        // LDS fragments in flight

  // S^T for the 64 keys of a K tile: two 32x32 blocks (chains interleaved)
  auto qk = [&](const uint4* kt, f32x16 (&s)[2]) {
    bf16x8 kb[kPfK];
#pragma unroll
    for (int f = 0; f < kPfK; ++f) kb[f] = kfrag(kt, f);
#pragma unroll
    for (int f = 0; f < kQkMfma; ++f) {
      s[f & 1] = mfma32(kb[f % kPfK], qf[f >> 1], f < 2 ? f32x16{} : s[f & 1]);
      if (f + kPfK < kQkMfma) kb[f % kPfK] = kfrag(kt, f + kPfK);
    }
  };
  auto mask_tile = [&](int j, f32x16 (&s)[2]) {
    const int kv0 = j * kPrefBN;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (kv0 + 32 * blk + acc_row(e, g) > qi) s[blk][e] = -INFINITY;
  };
  auto tile_max = [&](const f32x16 (&s)[2]) {
    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int e = 0; e < 16; e += 2) mx = fmax3_(mx, s[blk][e], s[blk][e + 1]);
    return xor32_max(mx);
  };

  f32x16 oacc[kV / 32];
#pragma unroll
  for (int i = 0; i < kV / 32; ++i) oacc[i] = f32x16{};
  float m_ref = -INFINITY;   // reference max (raw score units) the probabilities are taken against
  float m_true = -INFINITY;  // running max of this lane's query's raw scores
  float l_part = 0.0f;       // this lane half's share of the softmax denominator (w.r.t. m_ref)
  float mx_cur = -INFINITY;  // max of the current tile's scores
  const float c2 = scale * kLog2e;

  // probability pair i (elements 2i, 2i+1 of the 32 scores a lane holds)
  auto prob_pair = [&](const f32x16 (&s)[2], uint32_t (&pk)[2][8], float moff, float& psum, int i) {
    const int blk = i >> 3, e = 2 * (i & 7);
    const float p0 = fast_exp2(fmaf(s[blk][e], c2, moff));
    const float p1 = fast_exp2(fmaf(s[blk][e + 1], c2, moff));
    psum += p0 + p1;
    pk[blk][i & 7] = pack_bf16x2(p0, p1);
  };
  auto pv_operand = [&](const uint32_t (&pk)[2][8], int jj) {
    const uint32_t* src = &pk[jj >> 1][4 * (jj & 1)];
    return as_bf16x8(make_uint4(src[0], src[1], src[2], src[3]));
  };
  auto probs = [&](const f32x16 (&s)[2], uint32_t (&pk)[2][8], float moff) {
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) prob_pair(s, pk, moff, psum, i);
    l_part += psum;
  };
  auto pv = [&](const uint4* vtile, const uint32_t (&pk)[2][8]) {
    bf16x8 vb[kPfV];
#pragma unroll
    for (int f = 0; f < kPfV; ++f) vb[f] = vfrag(vtile, f);
#pragma unroll
    for (int f = 0; f < kPvMfma; ++f) {
      oacc[f & 3] = mfma32(vb[f % kPfV], pv_operand(pk, f >> 2), oacc[f & 3]);
      if (f + kPfV < kPvMfma) vb[f % kPfV] = vfrag(vtile, f + kPfV);
    }
  };
  // Overlapped tile body: the 24 score MFMAs of S(j+1) = K(j+1) Q^T and the
  // 16 value MFMAs of O^T += V(j)^T P(j)^T are issued in one interleaved
  // sequence (kOvl), each with one LDS operand read kRing MFMAs ahead and a
  // share of the VALU work: the probabilities of S(j) (pair p = elements 2p,
  // 2p+1 of the 32 scores a lane holds; the value MFMAs of 16 keys jj need
  // pairs 4jj..4jj+3) and the row max of S(j+1). Scheduling barriers keep
  // the issue order.
  auto overlapped = [&](const uint4* kt, const uint4* vtile, const f32x16 (&cur)[2], f32x16 (&nxt)[2],
                        float moff, auto&& issue_copy) {
    uint32_t pk[2][8];
    float psum = 0.0f;
    float mx0 = -INFINITY, mx1 = -INFINITY;
    bf16x8 ring[kRing];
    auto fetch = [&](auto C) {
      constexpr int c = decltype(C)::value;
      if constexpr (kOvl[c].qk) return kfrag(kt, 2 * (kOvl[c].idx % 12) + kOvl[c].idx / 12);
      else return vfrag(vtile, kOvl[c].idx);
    };
    static_for<0, kRing>([&](auto C) { ring[C] = fetch(C); });
    static_for<0, kOvlLen>([&](auto C) {
      constexpr int c = decltype(C)::value;
      constexpr Ovl o = kOvl[c];
      if constexpr (o.qk) {
        constexpr int blk = o.idx / 12, kk = o.idx % 12;
        if constexpr (kk == 0) nxt[blk] = mfma32(ring[c % kRing], qf[kk], f32x16{});
        else nxt[blk] = mfma32(ring[c % kRing], qf[kk], nxt[blk]);
      } else {
        oacc[o.idx & 3] = mfma32(ring[c % kRing], pv_operand(pk, o.idx >> 2), oacc[o.idx & 3]);
      }
      if constexpr (c + kRing < kOvlLen) ring[c % kRing] = fetch(std::integral_constant<int, c + kRing>{});
      if constexpr (c % 4 == 0 && c / 4 < kStepCopies) issue_copy(c / 4);
      if constexpr (o.pair >= 0) prob_pair(cur, pk, moff, psum, o.pair);
      if constexpr (o.mx >= 0) {
        mx0 = fmax3_(mx0, nxt[0][4 * o.mx], nxt[0][4 * o.mx + 1]);
        mx0 = fmax3_(mx0, nxt[0][4 * o.mx + 2], nxt[0][4 * o.mx + 3]);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    l_part += psum;
#pragma unroll
    for (int e = 0; e < 16; e += 2) mx1 = fmax3_(mx1, nxt[1][e], nxt[1][e + 1]);
    mx_cur = xor32_max(__builtin_elementwise_maximum(mx0, mx1));
  };

  f32x16 sA[2], sB[2];

  // one tile step; P = j & 1 picks the ring buffers and the score registers
  auto step = [&](auto par, int j) {
    constexpr int P = decltype(par)::value;
    uint4* kdst = P ? K1 : K0;            // K(j+2) replaces K(j)
    uint4* vdst = P ? V0 : V1;            // V(j+1) replaces V(j-1)
    const uint4* kread = P ? K0 : K1;     // K(j+1)
    const uint4* vread = P ? V1 : V0;     // V(j)
    f32x16 (&cur)[2] = P ? sB : sA;
    f32x16 (&nxt)[2] = P ? sA : sB;
    const bool cp_k = j + 2 < nkt, cp_v = j + 1 < nkt;
    // the step's copies are spread over the overlapped body (one per four
    // MFMAs) so that their issue hides behind the matrix work
    const bool spread = j < nkt_w && j + 2 < nkt_w;
    if (!spread) {
      if (cp_k) dma_k(kdst, j + 2);
      if (cp_v) dma_v(vdst, j + 1);
    }
    if (j < nkt_w) {
      // [A] move the reference max when S(j) exceeds it by more than 2^8
      const bool need = (mx_cur - m_ref) * c2 > kRescaleLog2;
      if (__ballot(need)) {
        const float m_new = need ? mx_cur : m_ref;
        const float corr = need ? fast_exp2((m_ref - m_new) * c2) : 1.0f;
        m_ref = m_new;
        l_part *= corr;
#pragma unroll
        for (int i = 0; i < kV / 32; ++i) oacc[i] *= corr;
      }
      m_true = fmaxf(m_true, mx_cur);
      const float moff = -m_ref * c2;
      if (j + 2 < nkt_w) {
        // (here j + 2 < nkt_w <= nkt: both K(j+2) and V(j+1) are due)
        overlapped(kread, vread, cur, nxt, moff, [&](int c) { dma_one(c, kdst, j + 2, vdst, j + 1); });
      } else if (j + 1 < nkt_w) {
        // the next tile is the wave's masked diagonal tile: the same
        // interleaved body (its copies went out above), then the mask and
        // the max of the masked scores
        overlapped(kread, vread, cur, nxt, moff, [](int) {});
        mask_tile(j + 1, nxt);
        mx_cur = tile_max(nxt);
      } else {
        // the wave's last tile
        uint32_t pk[2][8];
        probs(cur, pk, moff);
        pv(vread, pk);
      }
    }
    wait_vmcnt<0>();
    __syncthreads();
  };

  // ---- prologue: K(0), V(0), K(1) into LDS; S(0) as soon as the queries and
  // K(0) have landed (the later copies, issued after them, may still be in
  // flight), then V(0) and K(1) before the first step ----
  dma_k(K0, 0);
  dma_v(V0, 0);
  if (nkt > 1) {
    dma_k(K1, 1);
    wait_vmcnt<kVtCopies + kKcCopies + kKsCopies>();
  } else {
    wait_vmcnt<kVtCopies>();
  }
  // a bare barrier: __syncthreads' fence would wait for every copy in flight
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  if (nkt_w > 0) {
    qk(K0, sA);
    if (nkt_w == 1) mask_tile(0, sA);
    mx_cur = tile_max(sA);
  }
  wait_vmcnt<0>();
  __syncthreads();   // V(0) and K(1) are in; K0 is refilled by the first step

  for (int j = 0; j < nkt; j += 2) {
    step(std::integral_constant<int, 0>{}, j);
    if (j + 1 < nkt) step(std::integral_constant<int, 1>{}, j + 1);
  }

  // ---- epilogue: block maxima of the raw row max and of |q_t|^2 for the
  // max-logit refinement first (the barrier it needs then has no stores to
  // wait for), then normalise, gate and store; the stores drain after the
  // waves end. The gate values of the lane's 64 output columns are loaded
  // first, all in flight together, behind the reduction ----
  const size_t t_row = static_cast<size_t>(a0 + (qvalid ? qi : 0));
  uint2 gates[kV / 32][4];
  if (gate && qvalid) {
    const uint16_t* gr = gate + (t_row * heads + head) * kV;
#pragma unroll
    for (int db = 0; db < kV / 32; ++db)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp)
        gates[db][grp] = *reinterpret_cast<const uint2*>(gr + 32 * db + 8 * grp + 4 * g);
  }
  float qn2 = 0.0f;
#pragma unroll
  for (int kk = 0; kk < kD / 16; ++kk)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = static_cast<float>(qf[kk][e]);
      qn2 = fmaf(x, x, qn2);
    }
  qn2 += __shfl_xor(qn2, 32, 64);
  float v = qvalid ? m_true : -INFINITY;
  v = wave_max(v);
  qn2 = wave_max(qvalid ? qn2 : 0.0f);
  float* red = reinterpret_cast<float*>(K0);   // the rings are idle after the loop
  float* redq = red + kAttnWaves;
  if (lane == 0) {
    red[wave] = v;
    redq[wave] = qn2;
  }
  __syncthreads();
  if (tid == 0) {
    float mm = red[0], mq = redq[0];
    for (int w = 1; w < kAttnWaves; ++w) {
      mm = fmaxf(mm, red[w]);
      mq = fmaxf(mq, redq[w]);
    }
    if (mm > -INFINITY) atomic_max_float(aux + head * kAuxStride, mm);
    atomic_max_float(aux + head * kAuxStride + 1, mq);
  }
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
          const uint2 gv = gates[db][grp];
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
      if (lse) lse[static_cast<size_t>(head) * ntok + t] = m_ref * scale + __logf(l_tot);
      rowmax[static_cast<size_t>(head) * ntok + t] = m_true;
    }
  }
}

// ---------------------------------------------------------------------------
// Max-logit refinement. The attention kernel's logits carry the bf16 rounding
// of K^C (relative error up to 2^-8 per element: 8 significant bits), so
// its maximum can be off by ~1e-3.
// Every logit satisfies |approx - exact| <= delta with
//   delta = (2^-8 * 1.01 + 3e-5) * max_t |q_t| * max_s |K_s|
// (bf16 rounding of K^C plus fp32 accumulation), hence the exact maximum E
// lies in [M - delta, M + delta] for the approximate maximum M, and its row
// has an approximate row max >= M - 2 delta. Two small launches:
//   rows : rows whose approximate row max reaches M - 2 delta are listed,
//          and for each, q_abs = [W_UK_h^T q^C_t, q^R_t] in fp32
//          (K^C_s . q^C_t = c_s . q_abs by associativity), stored as bf16 hi
//          and lo parts (about 16 significant bits together) in the order
//          the score kernel's MFMA operands are loaded;
//   score: every key of every listed row (its sequence, up to the row) is
//          scored against hi and lo with MFMAs over the shared [c^KV | k^S]
//          rows, fp32 accumulation, and the maximum taken.
// Too many candidates (near-ties, e.g. q = 0) fall back to M, which is then
// within delta of E.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float refine_threshold(const float* aux, int h, int heads, float* M_out) {
  const float M = aux[h * kAuxStride];
  const float qn = sqrtf(aux[h * kAuxStride + 1]);
  const float kn = sqrtf(aux[h * kAuxStride + 2] + aux[static_cast<size_t>(heads) * kAuxStride]);
  *M_out = M;
  return M - 2.0f * (1.01f / 256.0f + 3e-5f) * qn * kn;
}

constexpr int kRefRowSplit = 4;     // workgroups per head scanning row maxima

__device__ __forceinline__ int seq_of(const int32_t* cu, int nseq, int t) {
  int lo = 0, hi = nseq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

constexpr int kRowList = 64;   // rows one rows workgroup lists before its head falls back

// Grid (heads, kRefRowSplit). Workgroup (h, y) scans every kRefRowSplit-th
// 256-row block of head h's row maxima and, for each row t that reaches the
// threshold (fewer than kRefRows per head), forms q_abs: thread i takes
// columns 8 (i % 64) .. +7 over the W_UK_h rows 32 (i / 64) .. +31 (its slab
// is loaded once, all 32 loads in flight, and kept for every row), the four
// partial sums of a column are added in a fixed order. The rows of all heads
// take dense numbers from one counter. A head with too many rows folds the
// approximate maximum M in instead (its listed rows are still scored).
__global__ void __launch_bounds__(256) prefill_refine_rows_kernel(
    const int32_t* __restrict__ cu, int nseq, int heads, int64_t ntok, const float* __restrict__ rowmax,
    const float* __restrict__ aux, const uint16_t* __restrict__ q, const uint16_t* __restrict__ w, float scale,
    int32_t* __restrict__ cand, uint16_t* __restrict__ qx, int4* __restrict__ qmeta, float* __restrict__ max_logit,
    int qnorm, const uint16_t* __restrict__ qn_w, float qn_eps) {
  __shared__ int lst[kRowList], lst_a0[kRowList];
  __shared__ float lst_r[kRowList];   // QK-norm factor of each listed row
  __shared__ int nl, n_acc, n_base;
  __shared__ float qcs[kRowList][kN];
  __shared__ __align__(16) float part[4][kR];
  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  float M;
  const float thr = refine_threshold(aux, h, heads, &M);
  if (!(M > -INFINITY)) return;
  // Seed the head slot with M - delta, a lower bound of the exact maximum
  // (which is among the scores formed below, so the result is unchanged):
  // the score kernel then only raises it with atomics near the maximum.
  if (blockIdx.y == 0 && tid == 0) atomic_max_float(max_logit + h, (M - 0.5f * (M - thr)) * scale);
  if (tid == 0) nl = 0;
  __syncthreads();
  // ---- scan: eight loads of a thread in flight at a time
  const int64_t step = 256 * static_cast<int64_t>(gridDim.y);
  for (int64_t t0 = tid + 256 * static_cast<int64_t>(blockIdx.y); t0 < ntok; t0 += 8 * step) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t t = t0 + u * step;
      v[u] = t < ntok ? rowmax[static_cast<size_t>(h) * ntok + t] : -INFINITY;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (v[u] >= thr) {
        const int k = atomicAdd(&nl, 1);
        if (k < kRowList) lst[k] = static_cast<int>(t0 + u * step);
      }
    }
  }
  __syncthreads();
  const int nfound = nl;
  if (nfound == 0) return;
  // ---- places among the head's kRefRows, and dense numbers, for all rows at once
  if (tid == 0) {
    const int c0 = atomicAdd(cand + kCandHeadCount + h, nfound);
    const int acc = max(0, min(min(nfound, kRowList), kRefRows - c0));
    n_acc = acc;
    n_base = acc > 0 ? atomicAdd(cand, acc) : 0;
    if (nfound > kRowList || c0 + nfound > kRefRows) atomic_max_float(max_logit + h, M * scale);   // fallback
  }
  __syncthreads();
  const int acc = n_acc, base = n_base;
  if (acc == 0) return;
  // ---- the W_UK_h slab of this thread and the queries of every accepted row, all loads in flight
  const int cg = tid & 63, kg = tid >> 6;
  uint4 wv[32];
  {
    const uint16_t* wr = w + (static_cast<size_t>(h) * (kN + kV) + 32 * kg) * kR + 8 * cg;
#pragma unroll
    for (int u = 0; u < 32; ++u) wv[u] = ldg16(wr + static_cast<size_t>(u) * kR);
  }
  if (tid < acc) {
    lst_a0[tid] = cu[seq_of(cu, nseq, lst[tid])];
    lst_r[tid] = qnorm ? qnorm_scale(qnorm_sumsq_row(q + (static_cast<size_t>(lst[tid]) * heads + h) * kD), qn_eps)
                       : 1.0f;
  }
  __syncthreads();
  for (int i = tid; i < acc * kN; i += 256) {
    const int k = i / kN, e = i - k * kN;
    const float x = bf16_to_f32(q[(static_cast<size_t>(lst[k]) * heads + h) * kD + e]);
    qcs[k][e] = qnorm ? qnorm_value(x, lst_r[k], qn_w, e) : x;
  }
  __syncthreads();
  const size_t plane = static_cast<size_t>(heads) * kRefRows * (kR + kS);
  for (int k = 0; k < acc; ++k) {
    const int t = lst[k], n = base + k;
    {
      float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        const float x = qcs[k][32 * kg + u];
        const uint32_t* w4 = &wv[u].x;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[2 * e] = fmaf(x, bf16lo(w4[e]), a[2 * e]);
          a[2 * e + 1] = fmaf(x, bf16hi(w4[e]), a[2 * e + 1]);
        }
      }
      float4* dst = reinterpret_cast<float4*>(&part[kg][8 * cg]);
      dst[0] = make_float4(a[0], a[1], a[2], a[3]);
      dst[1] = make_float4(a[4], a[5], a[6], a[7]);
    }
    __syncthreads();
    // Operand order: group n / 32, k-step kk = col / 16, lane 32 (col / 8 % 2)
    // + n % 32, element col % 8; hi and lo are separate planes.
    auto at = [&](int col) {
      return ((static_cast<size_t>(n >> 5) * ((kR + kS) / 16) + col / 16) * 64 + 32 * ((col >> 3) & 1) + (n & 31)) *
                 8 + (col & 7);
    };
    for (int col = tid; col < kR; col += 256) {
      const float v = (part[0][col] + part[1][col]) + (part[2][col] + part[3][col]);
      const uint16_t vh = f32_to_bf16(v);
      qx[at(col)] = vh;
      qx[plane + at(col)] = f32_to_bf16(v - bf16_to_f32(vh));
    }
    if (tid < kS) {   // q^R is bf16 already (normalised: rounded to bf16 as in the attention kernel)
      const uint16_t xr = q[(static_cast<size_t>(t) * heads + h) * kD + kN + tid];
      qx[at(kR + tid)] = qnorm ? f32_to_bf16(qnorm_value(bf16_to_f32(xr), lst_r[k], qn_w, kN + tid)) : xr;
      qx[plane + at(kR + tid)] = 0;
    }
    if (tid == 0) qmeta[n] = make_int4(t, lst_a0[k], h, 0);
    __syncthreads();   // part is rewritten for the next row
  }
}

constexpr int kScoreBlocks = 512;

// Grid (kScoreBlocks), persistent over units (group of 32 listed rows, 128
// consecutive keys). A unit's B operands (the group's q_abs hi and lo planes,
// 72 KB) are copied into LDS once; wave w then scores keys 32 w .. +31 of the
// unit: S = [c^KV | k^S]_keys (hi + lo)^T with 32x32x16 bf16 MFMAs (A: key
// rows from memory, loaded in three batches of 12 k-steps ahead of their
// MFMAs), and each listed row's maximum over its keys (same sequence, up to
// the row) is folded into the head's max logit. Units whose keys no listed
// row of the group reaches are skipped.
__global__ void __launch_bounds__(256) prefill_refine_score_kernel(
    const uint16_t* __restrict__ ckv, const uint16_t* __restrict__ ks, int64_t ntok, int heads,
    const int32_t* __restrict__ cand, const uint16_t* __restrict__ qx, const int4* __restrict__ qmeta, float scale,
    float* __restrict__ max_logit) {
  constexpr int kSteps = (kR + kS) / 16;   // 36
  __shared__ __align__(16) uint4 bl[2][kSteps * 64];   // [hi | lo][k-step][lane]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int ntot = min(cand[0], heads * kRefRows);
  if (ntot == 0) return;
  const int ncg = (ntot + 31) / 32;
  const int64_t nkb = (ntok + 127) / 128;
  const int64_t units = nkb * ncg;
  const size_t plane = static_cast<size_t>(heads) * kRefRows * (kR + kS);
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
    const int cgp = static_cast<int>(u / nkb);
    const int64_t kb0 = 128 * (u - static_cast<int64_t>(cgp) * nkb);
    const int n = 32 * cgp + l32;
    const bool nvalid = n < ntot;
    const int4 mt = qmeta[nvalid ? n : 0];
    const int t = mt.x, a0 = mt.y, h = mt.z;
    const int64_t k0 = kb0 + 32 * wave;
    const bool hit = nvalid && a0 <= k0 + 31 && t >= k0 && k0 < ntok;
    // block-uniform skip; the barrier also orders the previous unit's reads
    // of bl before this unit's writes
    if (!__syncthreads_or(hit ? 1 : 0)) continue;
    {
      const uint4* src = reinterpret_cast<const uint4*>(qx) + static_cast<size_t>(cgp) * kSteps * 64;
      const uint4* srl = reinterpret_cast<const uint4*>(qx + plane) + static_cast<size_t>(cgp) * kSteps * 64;
      uint4 x[2 * kSteps * 64 / 256];
#pragma unroll
      for (int i = 0; i < kSteps * 64 / 256; ++i) {
        x[i] = src[tid + 256 * i];
        x[kSteps * 64 / 256 + i] = srl[tid + 256 * i];
      }
#pragma unroll
      for (int i = 0; i < kSteps * 64 / 256; ++i) {
        bl[0][tid + 256 * i] = x[i];
        bl[1][tid + 256 * i] = x[kSteps * 64 / 256 + i];
      }
    }
    __syncthreads();
    if (__ballot(hit) == 0) continue;
    const int64_t s = min(k0 + l32, ntok - 1);   // this lane's key (A row)
    const uint16_t* crow = ckv + s * kR + 8 * g;
    const uint16_t* srow = ks + s * kS + 8 * g;
    f32x16 acc = f32x16{};
    static_for<0, 3>([&](auto bb) {
      constexpr int k0b = 12 * decltype(bb)::value;
      uint4 av[12];
      static_for<0, 12>([&](auto uu) {
        constexpr int kk = k0b + decltype(uu)::value;
        av[uu] = kk < kR / 16 ? ldg16(crow + 16 * kk) : ldg16(srow + 16 * (kk - kR / 16));
      });
      static_for<0, 12>([&](auto uu) {
        constexpr int kk = k0b + decltype(uu)::value;
        acc = mfma32(as_bf16x8(av[uu]), as_bf16x8(bl[0][kk * 64 + lane]), acc);
        acc = mfma32(as_bf16x8(av[uu]), as_bf16x8(bl[1][kk * 64 + lane]), acc);
      });
      __builtin_amdgcn_sched_group_barrier(0x020, 12, decltype(bb)::value);
      __builtin_amdgcn_sched_group_barrier(0x100, 24, decltype(bb)::value);
      __builtin_amdgcn_sched_group_barrier(0x008, 24, decltype(bb)::value);
    });
    float best = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t key = k0 + acc_row(e, g);
      if (key >= a0 && key <= t && key < ntok) best = fmaxf(best, acc[e]);
    }
    best = fmaxf(best, __shfl_xor(best, 32, 64));
    // Atomics only where they raise the slot (seeded with a lower bound of
    // the exact maximum by the rows kernel): its value only grows, so a stale
    // read can only cost an extra atomic. (One atomic per row and item on
    // the few dozen head slots would serialise in the L2.)
    if (g == 0 && nvalid && best > -INFINITY) {
      const float v = best * scale;
      if (v > *reinterpret_cast<volatile const float*>(max_logit + h)) atomic_max_float(max_logit + h, v);
    }
  }
}

hipError_t launch_prefill_bf16(int heads, float scale, bool out_bf16, const void* q, const void* ckv,
                               const void* ks, const void* w_kv_b, const void* gate, const int32_t* cu,
                               int nseq, int64_t ntok, void* out, float* lse, float* max_logit,
                               bool init_max_logit, void* ws, hipStream_t st, const QNorm& qn) {
  const PrefillWs L = prefill_ws_layout(heads, ntok, nseq);
  const int qnorm = qn.on ? 1 : 0;
  const uint16_t* qn_w = static_cast<const uint16_t*>(qn.w);
  char* base = static_cast<char*>(ws);
  uint16_t* kc = reinterpret_cast<uint16_t*>(base + L.kc);
  uint16_t* vt = reinterpret_cast<uint16_t*>(base + L.vt);
  uint16_t* ksp = reinterpret_cast<uint16_t*>(base + L.ksp);
  int32_t* pcu = reinterpret_cast<int32_t*>(base + L.pcu);
  int32_t* order = reinterpret_cast<int32_t*>(base + L.order);
  int32_t* toff = reinterpret_cast<int32_t*>(base + L.toff);
  int32_t* hdr = reinterpret_cast<int32_t*>(base + L.hdr);
  float* rowmax = reinterpret_cast<float*>(base + L.rowmax);
  float* aux = reinterpret_cast<float*>(base + L.aux);
  int32_t* cand = reinterpret_cast<int32_t*>(base + L.cand);

  {
    TimedScope ts_("prefill_plan", st);
    hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(kPlanThreads), 0, st, cu, nseq, pcu, order, toff, hdr, heads, aux,
                       cand, init_max_logit ? max_logit : nullptr);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  {
    const int64_t ex_items = (L.npad_max / kExRows + kExGroupRows - 1) / kExGroupRows *
                             ((heads + kExGroupHeads - 1) / kExGroupHeads) * kExGroup;
    TimedScope ts_("prefill_expand", st);
    hipLaunchKernelGGL(prefill_expand_kernel, dim3(static_cast<unsigned>((ex_items + 7) / 8 * 8)), dim3(kExThreads), 0,
                       st, static_cast<const uint16_t*>(ckv), static_cast<const uint16_t*>(w_kv_b), cu, nseq, pcu,
                       hdr, L.npad_max, ntok, heads, static_cast<const uint16_t*>(ks), kc, vt, ksp, aux);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  // upper bound on query tiles: sum over sequences of ceil(L/128) <= ntok/128 + nseq;
  // 8 XCDs with up to ceil(heads / 8) heads (or items) each
  const int64_t tiles_max = (ntok + kPrefBM - 1) / kPrefBM + nseq;
  const int64_t grid = 8 * tiles_max * ((heads + 7) / 8);
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  // Heads interleaved per XCD group: as many as keep the K and V that all
  // eight XCDs' groups read within about 96 MB (the last-level cache holds
  // 256 MB), between 2 and 12. Measured at 96 heads: at T = 4096 the rule's 6
  // is 2-4 % faster than 2 and as fast as 12 with a third less traffic; at
  // T = 8192 and 16384 groups of 6 and 3 equal 2, while 12 is 5 % and 12 %
  // slower.
  const int64_t kv_head_bytes = ntok * (kN + kV) * 2;
  const int hgroup = static_cast<int>(std::min<int64_t>(12, std::max<int64_t>(2, (int64_t{96} << 20) /
                                                                                     (8 * kv_head_bytes))));
  if (out_bf16) {
    {
      TimedScope ts_("prefill_attn", st);
      hipLaunchKernelGGL(prefill_attn_kernel<true>, dim3(static_cast<unsigned>(grid)), dim3(kAttnThreads), 0, st,
                         static_cast<const uint16_t*>(q), ksp,
                         static_cast<const uint16_t*>(gate), cu, pcu, order, toff, hdr, nseq, heads, ntok,
                         L.npad_max, kc, vt, scale, out, lse, rowmax, aux, qnorm, qn_w, qn.eps, hgroup);
    }
  } else {
    {
      TimedScope ts_("prefill_attn", st);
      hipLaunchKernelGGL(prefill_attn_kernel<false>, dim3(static_cast<unsigned>(grid)), dim3(kAttnThreads), 0, st,
                         static_cast<const uint16_t*>(q), ksp,
                         static_cast<const uint16_t*>(gate), cu, pcu, order, toff, hdr, nseq, heads, ntok,
                         L.npad_max, kc, vt, scale, out, lse, rowmax, aux, qnorm, qn_w, qn.eps, hgroup);
    }
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  uint16_t* qx = reinterpret_cast<uint16_t*>(base + L.qx);
  int4* qmeta = reinterpret_cast<int4*>(base + L.qmeta);
  {
    TimedScope ts_("prefill_refine_rows", st);
    hipLaunchKernelGGL(prefill_refine_rows_kernel, dim3(heads, kRefRowSplit), dim3(256), 0, st, cu, nseq, heads, ntok,
                       rowmax, aux, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(w_kv_b), scale,
                       cand, qx, qmeta, max_logit, qnorm, qn_w, qn.eps);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    TimedScope ts_("prefill_refine_score", st);
    hipLaunchKernelGGL(prefill_refine_score_kernel, dim3(kScoreBlocks), dim3(256), 0, st,
                       static_cast<const uint16_t*>(ckv), static_cast<const uint16_t*>(ks), ntok, heads, cand, qx,
                       qmeta, scale, max_logit);
  }
  return hipGetLastError();
}

}  // namespace mla
