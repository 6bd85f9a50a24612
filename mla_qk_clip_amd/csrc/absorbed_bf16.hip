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
//
// The per-head max logit is refined to the exact value: the split kernel
// bounds the bf16 rounding error of every 32-row tile's logits (from the
// tile's largest row norm) and keeps the tiles that could hold the maximum;
// the refine kernel re-scores those in fp32.
#include "mla_common.h"
#include "mla_internal.h"
#include "timing.h"

namespace mla {

constexpr int kW = kR + kS;  // 576 values per cache row

// P[v] = sum of visible rows of the virtual sequences before v; virtual
// sequence v = b * tq + i sees rows 0 .. lens[b] - tq + i of cache[b].
// One 256-thread block: per-thread chunk sums, an inclusive Hillis-Steele
// scan of the 256 sums in LDS (8 steps), then each thread writes its chunk's
// prefixes. Also clears the fix-up count.
__device__ void absorbed_prefix_block(const int32_t* __restrict__ lens, int tq, int64_t bt,
                                      int64_t* __restrict__ P, int32_t* __restrict__ nflag) {
  __shared__ int64_t sums[256];
  const int tid = threadIdx.x;
  const int64_t chunk = (bt + 255) / 256;
  const int64_t v0 = tid * chunk, v1 = min(bt, v0 + chunk);
  auto rows_of = [&](int64_t v) { return static_cast<int64_t>(lens[v / tq] - tq + static_cast<int>(v % tq) + 1); };
  int64_t s = 0;
  for (int64_t v = v0; v < v1; ++v) s += rows_of(v);
  sums[tid] = s;
  __syncthreads();
#pragma unroll
  for (int off = 1; off < 256; off <<= 1) {
    const int64_t t = tid >= off ? sums[tid - off] : 0;
    __syncthreads();
    sums[tid] += t;
    __syncthreads();
  }
  if (tid == 255) {
    P[bt] = sums[255];
    *nflag = 0;
  }
  int64_t acc = sums[tid] - s;
  for (int64_t v = v0; v < v1; ++v) {
    P[v] = acc;
    acc += rows_of(v);
  }
}

// q_abs[v][h][r] = sum_k w_kv_b[h*256 + k][r] * q[v][h][k]  (r < 512) as a
// bf16 MFMA product [64 v x 128 k] x [128 k x 128 r] per workgroup; the W_UK_h
// tile sits row-major in LDS and is read as the k-major operand with the
// LDS transpose read. q_abs[v][h][512 + s] = q[v][h][128 + s].
// Grid (heads, 4 column chunks of 128); 4 waves; virtual sequences in chunks of 64.
constexpr int kAqLd = 128 + 8;

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint16_t lds_u16;

// Transpose read (gfx950 ds_read_b64_tr_b16): within each group of 16 lanes,
// lane i passes the address of element (k0 + i/4, m0 + 4*(i%4)) of a
// row-major [k][m] tile and receives the column m0 + i at rows k0 .. k0+3.
__device__ __forceinline__ v4s lds_tr4(const lds_u16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p);
}
__device__ __forceinline__ bf16x8 cat_bf16(v4s lo, v4s hi) {
  typedef short v8s __attribute__((ext_vector_type(8)));
  const v8s x = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, x);
}

__global__ void __launch_bounds__(256) absorb_q_kernel(const uint16_t* __restrict__ q,
                                                       const uint16_t* __restrict__ w, int bt, int heads,
                                                       uint16_t* __restrict__ qabs, const int32_t* __restrict__ lens,
                                                       int tq, int64_t* __restrict__ P, int32_t* __restrict__ nflag,
                                                       float* __restrict__ ml_init, float* __restrict__ qn2,
                                                       float* __restrict__ hmax, uint16_t* __restrict__ qlo,
                                                       int qnorm, const uint16_t* __restrict__ qn_w, float qn_eps) {
  __shared__ __align__(16) uint16_t Wt[kN * kAqLd];
  __shared__ float qsq[2][64];
  __shared__ float qrs[64];   // QK-norm factor of each virtual sequence of the chunk
  const int h = blockIdx.x, rc = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  // W_UK_h rows k (128) x columns r in [128 rc, 128 rc + 128): all eight
  // 16-byte loads of a thread in flight before the LDS stores
  {
    uint4 wv[kN * 16 / 256];
#pragma unroll
    for (int j = 0; j < kN * 16 / 256; ++j) {
      const int c = tid + 256 * j, k = c >> 4, part = c & 15;
      wv[j] = ldg16(w + (static_cast<size_t>(h) * 256 + k) * kR + 128 * rc + 8 * part);
    }
#pragma unroll
    for (int j = 0; j < kN * 16 / 256; ++j) {
      const int c = tid + 256 * j, k = c >> 4, part = c & 15;
      *reinterpret_cast<uint4*>(Wt + k * kAqLd + 8 * part) = wv[j];
    }
  }
  if (h == 0 && rc == 0) {
    absorbed_prefix_block(lens, tq, bt, P, nflag);
    // max-logit slots start at -inf unless the caller accumulates into them
    if (ml_init && tid < heads) ml_init[tid] = -INFINITY;
    // state of the max-logit refinement (written by later kernels only)
    for (int i = tid; i < heads; i += 256) hmax[i] = -INFINITY;
  }
  __syncthreads();
  const lds_u16* wl = (const lds_u16*)(Wt);
  const int vb = wave & 1;          // which 32 virtual sequences of the 64-chunk
  const int rb0 = 2 * (wave >> 1);  // two 32-column blocks
  float qmax2 = 0.0f;
  for (int v0 = 0; v0 < bt; v0 += 64) {
    const int v = v0 + 32 * vb + l32;
    const bool vv = v < bt;
    f32x16 acc[2] = {f32x16{}, f32x16{}};
    uint4 qv[kN / 16];
#pragma unroll
    for (int kk = 0; kk < kN / 16; ++kk)
      qv[kk] = vv ? ldg16(q + (static_cast<size_t>(v) * heads + h) * kD + 16 * kk + 8 * g) : make_uint4(0, 0, 0, 0);
    if (qnorm) {
      // QK-norm variant: divide the head's query by the root mean square of
      // its D features (this lane half's q^C and q^R units, plus the other
      // half's sum), multiply by the weight, round to bf16
      uint4 qr[kS / 16];
#pragma unroll
      for (int j = 0; j < kS / 16; ++j)
        qr[j] = vv ? ldg16(q + (static_cast<size_t>(v) * heads + h) * kD + kN + 16 * j + 8 * g) : make_uint4(0, 0, 0, 0);
      float ss = 0.0f;
      auto acc_sq = [&](const uint4& u) {
        const uint32_t* w4 = &u.x;
#pragma unroll
        for (int i = 0; i < 4; ++i) ss = fmaf(bf16hi(w4[i]), bf16hi(w4[i]), fmaf(bf16lo(w4[i]), bf16lo(w4[i]), ss));
      };
#pragma unroll
      for (int kk = 0; kk < kN / 16; ++kk) acc_sq(qv[kk]);
#pragma unroll
      for (int j = 0; j < kS / 16; ++j) acc_sq(qr[j]);
      const float r = vv ? 1.0f / sqrtf((ss + __shfl_xor(ss, 32, 64)) / static_cast<float>(kD) + qn_eps) : 0.0f;
      auto norm_unit = [&](uint4& u, int f0) {
        uint32_t* w4 = &u.x;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float w0 = qn_w ? bf16_to_f32(qn_w[f0 + 2 * i]) : 1.0f;
          const float w1 = qn_w ? bf16_to_f32(qn_w[f0 + 2 * i + 1]) : 1.0f;
          w4[i] = pack_bf16x2(bf16lo(w4[i]) * r * w0, bf16hi(w4[i]) * r * w1);
        }
      };
#pragma unroll
      for (int kk = 0; kk < kN / 16; ++kk) norm_unit(qv[kk], 16 * kk + 8 * g);
      if (wave < 2 && g == 0) qrs[32 * vb + l32] = r;   // waves 0 and 1 hold the chunk's 64 rows
    }
#pragma unroll
    for (int kk = 0; kk < kN / 16; ++kk) {
      const bf16x8 a = as_bf16x8(qv[kk]);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int mb = 32 * (rb0 + j) + 16 * ((lane >> 4) & 1);
        const int i = lane & 15;
        const lds_u16* p0 = wl + (16 * kk + 8 * g + (i >> 2)) * kAqLd + mb + 4 * (i & 3);
        const bf16x8 b = cat_bf16(lds_tr4(p0), lds_tr4(p0 + 4 * kAqLd));
        acc[j] = mfma32(a, b, acc[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int vr = v0 + 32 * vb + acc_row(e, g);
        if (vr < bt) {
          // q_abs in bf16 for the stream, and its rounding residual (in bf16)
          // for the max-logit refinement
          const uint16_t hi = f32_to_bf16(acc[j][e]);
          const size_t col = (static_cast<size_t>(vr) * heads + h) * kR + 128 * rc + 32 * (rb0 + j) + l32;
          qabs[(static_cast<size_t>(vr) * heads + h) * kW + 128 * rc + 32 * (rb0 + j) + l32] = hi;
          qlo[col] = f32_to_bf16(acc[j][e] - bf16_to_f32(hi));
        }
      }
    if (qnorm) __syncthreads();   // qrs
    // q^R (normalised and rounded to bf16 under the QK-norm variant)
    auto qr_value = [&](int row, int s) {
      const uint16_t x = q[(static_cast<size_t>(v0 + row) * heads + h) * kD + kN + s];
      if (!qnorm) return x;
      return f32_to_bf16(bf16_to_f32(x) * qrs[row] * (qn_w ? bf16_to_f32(qn_w[kN + s]) : 1.0f));
    };
    if (rc == 0) {
      for (int e = tid; e < 64 * kS; e += 256) {
        const int vr = v0 + e / kS, s = e % kS;
        if (vr < bt) qabs[(static_cast<size_t>(vr) * heads + h) * kW + kR + s] = qr_value(e / kS, s);
      }
    }
    // squared norm of this block's 128 rounded q_abs entries per virtual
    // sequence: sum over the lane's two columns, then over the 32 lanes of
    // each half-wave (which share their rows), then over the two waves that
    // hold the same sequences
    float sq[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float a = bf16_to_f32(f32_to_bf16(acc[0][e])), b = bf16_to_f32(f32_to_bf16(acc[1][e]));
      sq[e] = fmaf(a, a, b * b);
    }
#pragma unroll
    for (int o = 1; o < 32; o <<= 1)
#pragma unroll
      for (int e = 0; e < 16; ++e) sq[e] += __shfl_xor(sq[e], o, 64);
    if (l32 == 0) {
#pragma unroll
      for (int e = 0; e < 16; ++e) qsq[wave >> 1][32 * vb + acc_row(e, g)] = sq[e];
    }
    __syncthreads();
    if (tid < 64 && v0 + tid < bt) {
      float s2 = qsq[0][tid] + qsq[1][tid];
      if (rc == 0) {
#pragma unroll 8
        for (int s = 0; s < kS; ++s) {
          const float x = bf16_to_f32(qr_value(tid, s));
          s2 = fmaf(x, x, s2);
        }
      }
      qmax2 = fmaxf(qmax2, s2);
    }
    __syncthreads();
  }
  // max over the virtual sequences; the sum over the four column blocks of
  // these maxima bounds every ||q_abs||^2 of the head
  if (wave == 0) {
    qmax2 = wave_max(qmax2);
    if (lane == 0) qn2[h * 4 + rc] = qmax2;
  }
}

// ---------------------------------------------------------------------------
// Split kernel. Workgroup = 4 waves; waves 0-2 each own 32 heads (head block
// 3*blockIdx.y + wave), wave 3 is the loader. The workgroup's rows are visited
// in tiles of 32 rows, segment (virtual sequence) by segment. The loader
// streams every tile straight from HBM into a ring of kStages LDS stages
// (global_load_lds, 16 bytes per lane, no registers), two tiles ahead of the
// compute; one barrier per tile.
// LDS tile layout: [32 rows][73 chunks of 8 bf16] (72 data chunks and one pad
// chunk per row, so rows are 36 banks apart and both read patterns below are
// free of bank conflicts). A wave-wide copy fills 64 consecutive chunk slots;
// lanes that land on a pad slot fetch a harmless valid chunk.
// A compute wave keeps its heads' q_abs as MFMA operands in registers, forms
// S^T = C Q^T (each lane owns one head column; rows of C read as b128) and
// accumulates O_lat^T = C^T P^T with C^T read through the LDS transpose read.
// The softmax takes every probability against a fixed reference, the first
// tile's max of the segment, so the accumulators are never rescaled; a head
// whose later logits exceed the reference by more than 64 in exp2 units is
// flagged (and counted in nflag) and its segment is recomputed by the fix-up
// kernel.
// Partials per (workgroup, virtual sequence) slot and head:
//   part_o[slot][h][r] = sum_j p_j c_j[r] (relative to the reference max),
//   part_ml[slot][h] = {reference max (raw), denominator, true raw max, flag}.
// ---------------------------------------------------------------------------
// Bound on |streamed - exact| logit per unit of ||q_abs|| * ||row||: bf16
// rounding of q_abs (unit roundoff 2^-8, with 1% slack for the fp32
// products that formed it) plus fp32 accumulation over 576 products.
constexpr float kDecErrCoef = 1.01f / 256.0f + 4e-5f;

constexpr int kChunks = kW / 8;                       // 72 data chunks of 16 bytes per row
constexpr int kRowSlots = kChunks + 1;                // 73 slots per LDS row (one pad)
constexpr int kTileSlots = kDecRows * kRowSlots;      // 2336
constexpr int kDmaCopies = (kTileSlots + 63) / 64;    // 37 wave-wide 1 KB copies per tile
constexpr int kTileBytes = kDmaCopies * 1024;         // 37888 bytes per stage
constexpr int kStages = 3;

struct TileCursor {
  int64_t vs;       // virtual sequence of the current tile
  int64_t pos;      // global start row of the current tile
  int64_t seg_end;  // global end of the current segment (within the workgroup range)
  int64_t hi;
};

__device__ __forceinline__ void cursor_init(TileCursor& c, const int64_t* P, int64_t bt, int64_t lo, int64_t hi) {
  int64_t vlo = 0, vhi = bt - 1;
  while (vlo < vhi) {
    const int64_t mid = (vlo + vhi + 1) >> 1;
    if (P[mid] <= lo) vlo = mid; else vhi = mid - 1;
  }
  while (P[vlo + 1] <= lo) ++vlo;
  c.vs = vlo;
  c.pos = lo;
  c.hi = hi;
  c.seg_end = min(hi, P[vlo + 1]);
}
__device__ __forceinline__ void cursor_next(TileCursor& c, const int64_t* P) {
  c.pos = min(c.pos + kDecRows, c.seg_end);
  if (c.pos >= c.seg_end && c.pos < c.hi) {
    while (P[c.vs + 1] <= c.pos) ++c.vs;
    c.seg_end = min(c.hi, P[c.vs + 1]);
  }
}

// vmcnt-only wait (expcnt and lgkmcnt left at their maxima), gfx9 encoding

struct SplitState {
  bf16x8 qf[kW / 16];
  f32x16 oacc[kR / 32];
  float m_ref, m_true, l_part;
  bool overflow, first;
};

// Scores, softmax weights and the latent accumulation for one tile in `tile`.
// Returns the tile's approximate max logit of the lane's head.
__device__ __forceinline__ float split_compute(const uint16_t* tile, int nrows, int lane, float c2, SplitState& S) {
  const int g = lane >> 5, l32 = lane & 31;
  const int i16 = lane & 15;
  const int mhalf = 16 * ((lane >> 4) & 1);
  const char* tb = reinterpret_cast<const char*>(tile);
  const lds_u16* tl = (const lds_u16*)(tile);
  // S^T = C Q^T with the LDS operand reads issued kPf k-steps ahead of their MFMA
  constexpr int kPf = 6;
  const uint4* arow = reinterpret_cast<const uint4*>(tb + 16 * (l32 * kRowSlots + g));
  uint4 af[kPf];
#pragma unroll
  for (int kk = 0; kk < kPf; ++kk) af[kk] = arow[2 * kk];
  f32x16 sacc = f32x16{};
#pragma unroll
  for (int kk = 0; kk < kW / 16; ++kk) {
    const bf16x8 a = as_bf16x8(af[kk % kPf]);
    if (kk + kPf < kW / 16) af[kk % kPf] = arow[2 * (kk + kPf)];
    sacc = mfma32(a, S.qf[kk], sacc);
  }
  // keep the reads kPf MFMAs ahead (the scheduler would otherwise sink them
  // next to their uses and expose the LDS latency on every MFMA)
  __builtin_amdgcn_sched_group_barrier(0x100, kPf, 0);
#pragma unroll
  for (int kk = 0; kk < kW / 16; ++kk) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
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
  if (S.first) S.m_ref = mx;
  S.m_true = fmaxf(S.m_true, mx);
  S.overflow = S.overflow || (mx - S.m_ref) * c2 > 64.0f;
  const float moff = -S.m_ref * c2;
  uint32_t pk[8];
  float psum = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; e += 2) {
    const float p0 = fast_exp2(fmaf(sacc[e], c2, moff));
    const float p1 = fast_exp2(fmaf(sacc[e + 1], c2, moff));
    psum += p0 + p1;
    pk[e >> 1] = pack_bf16x2(p0, p1);
  }
  S.l_part += psum;
  // O_lat^T += C^T P^T: 32 MFMAs (2 row halves x 16 latent blocks); the two
  // transpose reads of each operand are issued kPv MFMAs ahead
  constexpr int kPv = 4;
  const bf16x8 bp0 = as_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3]));
  const bf16x8 bp1 = as_bf16x8(make_uint4(pk[4], pk[5], pk[6], pk[7]));
  const lds_u16* rowp = tl + (4 * g + (i16 >> 2)) * (8 * kRowSlots) + mhalf + 4 * (i16 & 3);
  auto pv_ptr = [&](int m) { return rowp + (m >> 4) * 16 * (8 * kRowSlots) + 32 * (m & 15); };
  v4s t0[kPv], t1[kPv];
#pragma unroll
  for (int m = 0; m < kPv; ++m) {
    t0[m] = lds_tr4(pv_ptr(m));
    t1[m] = lds_tr4(pv_ptr(m) + 8 * (8 * kRowSlots));
  }
#pragma unroll
  for (int m = 0; m < 2 * (kR / 32); ++m) {
    const bf16x8 a = cat_bf16(t0[m % kPv], t1[m % kPv]);
    if (m + kPv < 2 * (kR / 32)) {
      t0[m % kPv] = lds_tr4(pv_ptr(m + kPv));
      t1[m % kPv] = lds_tr4(pv_ptr(m + kPv) + 8 * (8 * kRowSlots));
    }
    S.oacc[m & 15] = mfma32(a, (m >> 4) ? bp1 : bp0, S.oacc[m & 15]);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * kPv, 1);
#pragma unroll
  for (int m = 0; m < 2 * (kR / 32); ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
  }
  return mx;
}

// Wave 3 streams every tile of the workgroup into a ring of kStages LDS stages
// with direct global->LDS copies (37 wave-wide 1 KB copies per tile), two
// tiles ahead of the compute waves. It issues no other vector memory
// operations (so its vmcnt waits count copies only), its LDS reads of the
// ring are written in asm, and the compute waves never copy, so neither code
// path has to wait on the other's memory ops except through the explicit
// vmcnt wait and the barrier.
struct TileRec {
  int vs, row0, nrows;   // virtual sequence, first row within it, rows
};

__device__ __forceinline__ TileRec split_issue(uint16_t* ring, int stage, TileCursor& lc, const int64_t* P,
                                               const uint16_t* cache, int64_t cap, int tq, int lane) {
  const int b = static_cast<int>(lc.vs / tq);
  const int64_t row0 = lc.pos - P[lc.vs];
  const int64_t left = lc.seg_end - lc.pos;
  const int nrows = left < kDecRows ? static_cast<int>(left) : kDecRows;
  const TileRec rec{static_cast<int>(lc.vs), static_cast<int>(row0), nrows};
  const uint16_t* src = cache + (static_cast<size_t>(b) * cap + row0) * kW;
  char* dst = reinterpret_cast<char*>(ring) + stage * kTileBytes;
#pragma unroll
  for (int kc = 0; kc < kDmaCopies; ++kc) {
    const int slot = 64 * kc + lane;
    int r = slot / kRowSlots;
    int c = slot - r * kRowSlots;
    // pad slots, slots past the tile and rows past the segment fetch a valid
    // chunk of the tile's first row (finite; never used or masked)
    if (r >= nrows || c >= kChunks) {
      r = 0;
      c = 0;
    }
    __builtin_amdgcn_global_load_lds(src + r * kW + 8 * c,
                                     (__attribute__((address_space(3))) void*)(dst + 1024 * kc), 16, 0, 0);
  }
  cursor_next(lc, P);
  return rec;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Nine 16-byte LDS reads at addr + 16 k, k < 9, with their wait in the same
// asm block. Written this way because the compiler orders every LDS read of
// the ring behind all of the wave's outstanding global->LDS copies; these
// reads touch a stage whose copies have completed.
__device__ __forceinline__ void lds_read9(uint32_t addr, u32x4 (&x)[9]) {
  asm volatile(
      "ds_read_b128 %0, %9\n"
      "ds_read_b128 %1, %9 offset:16\n"
      "ds_read_b128 %2, %9 offset:32\n"
      "ds_read_b128 %3, %9 offset:48\n"
      "ds_read_b128 %4, %9 offset:64\n"
      "ds_read_b128 %5, %9 offset:80\n"
      "ds_read_b128 %6, %9 offset:96\n"
      "ds_read_b128 %7, %9 offset:112\n"
      "ds_read_b128 %8, %9 offset:128\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]),
        "=&v"(x[7]), "=&v"(x[8])
      : "v"(addr)
      : "memory");
}

// Largest row norm among the first nrows rows of an LDS tile. Lane l sums
// the squares of half of row l % 32 (36 of its 72 chunks); the halves are
// added, then the maximum is taken over the rows.
__device__ __forceinline__ float tile_max_row_norm(const uint16_t* tile, int nrows, int lane) {
  const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_u16*)tile)) +
                        16 * ((lane & 31) * kRowSlots + (kChunks / 2) * (lane >> 5));
  float s = 0.0f;
#pragma unroll
  for (int blk = 0; blk < kChunks / 2 / 9; ++blk) {
    u32x4 x[9];
    lds_read9(base + 16 * 9 * blk, x);
#pragma unroll
    for (int k = 0; k < 9; ++k) {
      // (bit-casting single elements of a vector would read element 0 with this compiler)
      const bf16x8 v = __builtin_bit_cast(bf16x8, x[k]);
      const bf16x2 v0 = __builtin_shufflevector(v, v, 0, 1), v1 = __builtin_shufflevector(v, v, 2, 3);
      const bf16x2 v2 = __builtin_shufflevector(v, v, 4, 5), v3 = __builtin_shufflevector(v, v, 6, 7);
      s = __builtin_amdgcn_fdot2_f32_bf16(v0, v0, s, false);
      s = __builtin_amdgcn_fdot2_f32_bf16(v1, v1, s, false);
      s = __builtin_amdgcn_fdot2_f32_bf16(v2, v2, s, false);
      s = __builtin_amdgcn_fdot2_f32_bf16(v3, v3, s, false);
    }
  }
  s += __shfl_xor(s, 32, 64);
  if ((lane & 31) >= nrows) s = 0.0f;
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) s = fmaxf(s, __shfl_xor(s, o, 64));
  return sqrtf(s);
}

// Workgroup barrier for the loader wave: the caller has already waited for
// exactly the copies the other waves need. (__syncthreads would also wait for
// the copies of the tile two ahead, which are not needed yet.) The compiler
// keeps memory accesses on their side of the asm statements.
__device__ __forceinline__ void loader_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Candidate list of one head in one split workgroup, kept by the lane that
// owns the head. lb is a lower bound of the head's exact max logit (the
// largest tile max minus its error bound so far); a tile can hold the exact
// maximum only if its max plus its error bound reaches lb, so entries below
// the current lb are dropped whenever the list fills up. cnt == kDecList + 1
// marks a list that overflowed with live entries.
struct CandEntry {
  int vsn;    // virtual sequence | rows << 24
  int row0;   // first row within the sequence
  float u;    // upper bound of the tile's exact max logit (raw)
};
__device__ __forceinline__ void cand_compact(CandEntry* list, int& cnt, float lb) {
  int j = 0;
  for (int k = 0; k < cnt; ++k) {
    const CandEntry e = list[k];
    if (e.u >= lb) list[j++] = e;
  }
  cnt = j;
}
__device__ __forceinline__ void cand_record(CandEntry* list, int& cnt, float& lb, float mx, float d, int vsn,
                                            int row0) {
  lb = fmaxf(lb, mx - d);
  const float u = mx + d;
  if (cnt > kDecList || u < lb) return;
  if (cnt == kDecList) {
    cand_compact(list, cnt, lb);
    if (cnt == kDecList) {
      cnt = kDecList + 1;
      return;
    }
  }
  list[cnt++] = CandEntry{vsn, row0, u};
}

__global__ void __launch_bounds__(256) absorbed_split_kernel(
    const uint16_t* __restrict__ cache, int64_t cap, int tq, int heads, int64_t bt,
    const int64_t* __restrict__ P, const uint16_t* __restrict__ qabs, float scale,
    float* __restrict__ part_o, float* __restrict__ part_ml, int32_t* __restrict__ nflag,
    const float* __restrict__ qn2, float* __restrict__ dlb, int32_t* __restrict__ dcnt, int4* __restrict__ dent) {
  __shared__ __align__(16) uint16_t ring[kStages * kTileBytes / 2];
  // largest row norm of the tile being computed (double-buffered), from the
  // loader to the compute waves
  __shared__ float tnorm[2];
  // per head of the block: candidate tiles for the max-logit refinement
  __shared__ CandEntry clist[kDecHeadsPerWg][kDecList];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int G = gridDim.x;
  const int64_t total = P[bt];
  const int64_t lo = total * blockIdx.x / G;
  const int64_t hi = total * (blockIdx.x + 1) / G;
  // the first head block writes the bounds of every head of an empty workgroup
  const bool rec = blockIdx.y == 0;
  if (lo >= hi) {
    // no rows: no bound and no candidates for any head
    if (rec) {
      for (int h = tid; h < heads; h += 256) {
        dlb[blockIdx.x * heads + h] = -INFINITY;
        dcnt[blockIdx.x * heads + h] = 0;
      }
    }
    return;
  }

  int ntiles = 0;
  {
    TileCursor c;
    cursor_init(c, P, bt, lo, hi);
    while (c.pos < hi) {
      ++ntiles;
      cursor_next(c, P);
    }
  }

  if (wave == 3) {
    // ---------------- loader ----------------
    // It also measures each tile the compute waves are working on (its
    // largest row norm, from LDS, while the next copies are in flight) and
    // leaves the result in tnorm for the compute waves.
    TileCursor lc;
    cursor_init(lc, P, bt, lo, hi);
    TileRec r0 = split_issue(ring, 0, lc, P, cache, cap, tq, lane);
    TileRec r1 = ntiles > 1 ? split_issue(ring, 1, lc, P, cache, cap, tq, lane) : TileRec{0, 0, 0};
    if (ntiles > 1) wait_vmcnt<kDmaCopies>(); else wait_vmcnt<0>();   // tile 0 landed
    loader_barrier();
    for (int i = 0; i < ntiles; ++i) {
      TileRec r2{0, 0, 0};
      if (i + 2 < ntiles) r2 = split_issue(ring, (i + 2) % kStages, lc, P, cache, cap, tq, lane);
      {
        const float kn = tile_max_row_norm(ring + (i % kStages) * (kTileBytes / 2), r0.nrows, lane);
        if (lane == 0) tnorm[i & 1] = kn;
      }
      r0 = r1;
      r1 = r2;
      // tile i+1 must have landed (and tnorm been written) before the barrier that ends tile i
      if (i + 2 < ntiles) wait_vmcnt<kDmaCopies>(); else wait_vmcnt<0>();
      __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
      loader_barrier();
    }
    return;
  }

  // ---------------- compute waves ----------------
  const int hb = 3 * blockIdx.y + wave;
  const int head = 32 * hb + l32;
  const bool active = 32 * hb < heads;
  const bool hvalid = active && head < heads;
  const float c2 = scale * kLog2e;
  // the head's logit error bound per unit row norm, and its candidate list
  const int hq = hvalid ? head : 0;
  const float qerr =
      kDecErrCoef * sqrtf((qn2[4 * hq] + qn2[4 * hq + 1]) + (qn2[4 * hq + 2] + qn2[4 * hq + 3]));
  CandEntry* clst = clist[32 * wave + l32];
  float clb = -INFINITY;
  int ccnt = 0;
  __syncthreads();   // tile 0

  TileCursor cur;
  cursor_init(cur, P, bt, lo, hi);
  int i = 0;   // global tile index of this workgroup
  SplitState S;
  while (cur.pos < hi) {
    // ---- one segment: the rows of virtual sequence cur.vs inside [lo, hi) ----
    const int64_t vs = cur.vs;
    const int64_t seg_end = cur.seg_end;
    const int64_t seg_p = P[vs];   // global index of the sequence's first visible row
    {
      const uint16_t* qrow = qabs + (static_cast<size_t>(vs) * heads + (hvalid ? head : 0)) * kW + 8 * g;
#pragma unroll
      for (int kk = 0; kk < kW / 16; ++kk)
        S.qf[kk] = as_bf16x8(hvalid ? ldg16(qrow + 16 * kk) : make_uint4(0, 0, 0, 0));
#pragma unroll
      for (int j = 0; j < kR / 32; ++j) S.oacc[j] = f32x16{};
    }
    // Fixed reference max per segment (the first tile's): probabilities
    // relative to it may exceed 1 but stay far inside the bf16 / fp32 range
    // unless a later logit exceeds it by more than 64 / c2 (p > 2^64; flagged,
    // and such segments are recomputed by the fix-up kernel).
    S.m_ref = 0.0f;
    S.m_true = -INFINITY;
    S.l_part = 0.0f;
    S.overflow = false;
    S.first = true;
    do {
      const int64_t left = seg_end - cur.pos;
      const int nrows = left < kDecRows ? static_cast<int>(left) : kDecRows;
      float mx = 0.0f;
      if (active) mx = split_compute(ring + (i % kStages) * (kTileBytes / 2), nrows, lane, c2, S);
      S.first = false;
      __syncthreads();
      // the finished tile into the head's candidate list for the max-logit
      // refinement, with the loader's row norm for its error bound
      if (hvalid && g == 0)
        cand_record(clst, ccnt, clb, mx, qerr * tnorm[i & 1], static_cast<int>(vs) | (nrows << 24),
                    static_cast<int>(cur.pos - seg_p));
      cursor_next(cur, P);
      ++i;
    } while (cur.pos < seg_end);

    // ---- the segment's partial ----
    if (hvalid) {
      const size_t slot = static_cast<size_t>(blockIdx.x) + static_cast<size_t>(vs);
      float* po = part_o + (slot * heads + head) * kR;
#pragma unroll
      for (int cbk = 0; cbk < kR / 32; ++cbk)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          const int r = 32 * cbk + 8 * grp + 4 * g;
          *reinterpret_cast<float4*>(po + r) = make_float4(S.oacc[cbk][4 * grp], S.oacc[cbk][4 * grp + 1],
                                                           S.oacc[cbk][4 * grp + 2], S.oacc[cbk][4 * grp + 3]);
        }
      const float l_tot = S.l_part + __shfl_xor(S.l_part, 32, 64);
      if (g == 0)
        *reinterpret_cast<float4*>(part_ml + (slot * heads + head) * 4) =
            make_float4(S.m_ref, l_tot, S.m_true, S.overflow ? 1.0f : 0.0f);
      if (__ballot(S.overflow) && lane == 0) atomicAdd(nflag, 1);
    }
  }
  // the head's bound and live candidates of this workgroup
  if (hvalid && g == 0) {
    if (ccnt <= kDecList) cand_compact(clst, ccnt, clb);
    const size_t o = static_cast<size_t>(blockIdx.x) * heads + head;
    dlb[o] = clb;
    dcnt[o] = ccnt;
    for (int k = 0; k < ccnt && k < kDecList; ++k) {
      const CandEntry e = clst[k];
      dent[o * kDecList + k] = make_int4(e.vsn & 0xffffff, e.row0, e.vsn >> 24, __float_as_int(e.u));
    }
  }
}

// ---------------------------------------------------------------------------
// Fix-up for segments whose logits outgrew the split kernel's fixed reference
// (a later logit above the first tile's max by more than 64 / c2, i.e. far
// outside normal attention statistics): recompute those (segment, head)
// partials with a plain online softmax that rescales as it goes. One
// workgroup per split workgroup; one wavefront per flagged head at a time.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) absorbed_fixup_kernel(
    const uint16_t* __restrict__ cache, int64_t cap, int tq, int heads, int64_t bt, int G,
    const int64_t* __restrict__ P, const uint16_t* __restrict__ qabs, float scale, float* __restrict__ part_o,
    float* __restrict__ part_ml, const int32_t* __restrict__ nflag) {
  if (*nflag == 0) return;   // nothing was flagged (the common case)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t total = P[bt];
  const int64_t lo = total * blockIdx.x / G;
  const int64_t hi = total * (blockIdx.x + 1) / G;
  if (lo >= hi) return;
  const float c2 = scale * kLog2e;
  TileCursor cur;
  cursor_init(cur, P, bt, lo, hi);
  while (cur.pos < hi) {
    const int64_t vs = cur.vs;
    const int64_t seg_beg = cur.pos, seg_end = cur.seg_end;
    const size_t slot = static_cast<size_t>(blockIdx.x) + static_cast<size_t>(vs);
    const int b = static_cast<int>(vs / tq);
    const uint16_t* cb = cache + static_cast<size_t>(b) * cap * kW;
    for (int h = wave; h < heads; h += 4) {
      float* ml = part_ml + (slot * heads + h) * 4;
      if (ml[3] == 0.0f) continue;
      // q_abs of this head, 9 features per lane
      float qa[kW / 64];
      const uint16_t* qrow = qabs + (static_cast<size_t>(vs) * heads + h) * kW;
#pragma unroll
      for (int j = 0; j < kW / 64; ++j) qa[j] = bf16_to_f32(qrow[lane + 64 * j]);
      float o[kR / 64];
#pragma unroll
      for (int j = 0; j < kR / 64; ++j) o[j] = 0.0f;
      float m = -INFINITY, l = 0.0f;
      for (int64_t r = seg_beg - P[vs]; r < seg_end - P[vs]; ++r) {
        const uint16_t* row = cb + static_cast<size_t>(r) * kW;
        float part = 0.0f;
        float cv[kR / 64];
#pragma unroll
        for (int j = 0; j < kW / 64; ++j) {
          const float x = bf16_to_f32(row[lane + 64 * j]);
          if (j < kR / 64) cv[j] = x;
          part = fmaf(qa[j], x, part);
        }
        const float sraw = wave_sum(part);
        const float m_new = fmaxf(m, sraw);
        const float corr = fast_exp2((m - m_new) * c2);
        const float p = fast_exp2((sraw - m_new) * c2);
        l = l * corr + p;
#pragma unroll
        for (int j = 0; j < kR / 64; ++j) o[j] = o[j] * corr + p * cv[j];
        m = m_new;
      }
      float* po = part_o + (slot * heads + h) * kR;
#pragma unroll
      for (int j = 0; j < kR / 64; ++j) po[lane + 64 * j] = o[j];
      if (lane == 0) {
        ml[0] = m;
        ml[1] = l;
        ml[2] = m;
        ml[3] = 0.0f;
      }
    }
    cur.pos = seg_end;
    if (cur.pos < hi) {
      while (P[cur.vs + 1] <= cur.pos) ++cur.vs;
      cur.seg_end = min(hi, P[cur.vs + 1]);
    }
  }
}

// ---------------------------------------------------------------------------
// Combine: merge the partials of each (virtual sequence, head) by log-sum-exp,
// then O~ = o_lat W_UV_h^T, gate, store, and the per-head approximate max logit.
// Grid (heads, ceil(bt / 16)); 256 threads.
// Phase 1: 16 threads per virtual sequence, thread `sub` owning the latent
// columns 4 sub + 64 e + j (e < 8, j < 4), so that one load instruction reads
// 256 contiguous bytes of a partial; partials are visited two at a time with
// all of their loads in flight. Splits that hold no rows (fewer rows than
// splits in total) wrote no partial and are skipped. o_lat goes to LDS as a
// pair of bf16 parts, hi = bf16(o) and lo = bf16(o - hi), which together
// carry about 16 significant bits.
// Phase 2: O~^T [128 d x 16 v] = W_UV_h [128 x 512] o_lat^T with 16x16x32 bf16
// MFMAs on both parts; wave w computes d in [32 w, 32 w + 32) and loads its
// W_UV_h operands at kernel start, so they arrive during phase 1.
// ---------------------------------------------------------------------------
constexpr int kCmbV = 16;

constexpr int kCmbLd = kR + 8;   // LDS row of the o_lat parts (16-byte pad)

// First cache row of split workgroup w (the split kernel's partition).
__device__ __forceinline__ int64_t split_lo(int64_t total, int w) { return total * w / kDecSplits; }

// The split workgroup whose rows contain `row`: the largest w with split_lo(w) <= row.
__device__ __forceinline__ int split_of_row(int64_t total, int64_t row) {
  int lo = 0, hi = kDecSplits - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (split_lo(total, mid) <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ float group16_max(float v) {
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

template <bool OUT_BF16>
__global__ void __launch_bounds__(256) absorbed_combine_kernel(
    const int64_t* __restrict__ P, int64_t bt, int heads, float scale, const float* __restrict__ part_o,
    const float* __restrict__ part_ml, const uint16_t* __restrict__ w, const uint16_t* __restrict__ gate,
    void* __restrict__ out, float* __restrict__ hmax) {
  __shared__ __align__(16) uint16_t ohi[kCmbV * kCmbLd];
  __shared__ __align__(16) uint16_t olo[kCmbV * kCmbLd];
  __shared__ float red[kCmbV];
  const int h = blockIdx.x;
  const int64_t v0 = static_cast<int64_t>(blockIdx.y) * kCmbV;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i16 = lane & 15, kq = lane >> 4;

  // W_UV_h rows d = 32 wave + 16 b + i16, k-slots 8 kq .. +7 of every 32-wide
  // step; the first half of the steps is loaded now (arriving during phase
  // 1), the second half when phase 2 starts.
  constexpr int kKs = kR / 32;
  const uint16_t* wrow = w + (static_cast<size_t>(h) * 256 + kN + 32 * wave + i16) * kR + 8 * kq;
  uint4 wop[2][kKs];
  static_for<0, 2>([&](auto b) {
    static_for<0, kKs / 2>([&](auto kk) { wop[b][kk] = ldg16(wrow + b * 16 * kR + 32 * kk); });
  });

  // ---- phase 1: o_lat of the workgroup's 16 virtual sequences ----
  // Online merge: partials are visited two at a time (all their loads in
  // flight together) against a running reference max M.
  const int vl = tid >> 4, sub = tid & 15;
  const int64_t vs = v0 + vl;
  const float c2 = scale * kLog2e;
  float acc[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) acc[e] = 0.0f;
  float den = 1.0f, Mt = -INFINITY;
  if (vs < bt) {
    const int64_t total = P[bt];
    const int wa = split_of_row(total, P[vs]);
    const int wb = split_of_row(total, P[vs + 1] - 1);
    auto nonempty = [&](int s) { return split_lo(total, s) < split_lo(total, s + 1); };
    float M = -INFINITY;
    den = 0.0f;
    const float* pb = part_o + static_cast<size_t>(h) * kR + 4 * sub;
    // split wa holds the sequence's first row, so the first pair is never empty
    for (int s = wa; s <= wb; s += 2) {
      const bool e0 = nonempty(s);
      const bool e1 = s + 1 <= wb && nonempty(s + 1);
      const size_t slot0 = (static_cast<size_t>(s) + vs) * heads + h;
      const size_t slot1 = slot0 + heads;
      float4 m0 = make_float4(-INFINITY, 0.f, -INFINITY, 0.f), m1 = m0;
      float4 x0[8], x1[8];
      if (e0) {
        m0 = *reinterpret_cast<const float4*>(part_ml + slot0 * 4);
        const float* p0 = pb + (static_cast<size_t>(s) + vs) * heads * kR;
#pragma unroll
        for (int e = 0; e < 8; ++e) x0[e] = *reinterpret_cast<const float4*>(p0 + 64 * e);
      }
      if (e1) {
        m1 = *reinterpret_cast<const float4*>(part_ml + slot1 * 4);
        const float* p1 = pb + (static_cast<size_t>(s) + 1 + vs) * heads * kR;
#pragma unroll
        for (int e = 0; e < 8; ++e) x1[e] = *reinterpret_cast<const float4*>(p1 + 64 * e);
      }
      Mt = fmaxf(Mt, fmaxf(m0.z, m1.z));
      const float mnew = fmaxf(M, fmaxf(m0.x, m1.x));
      if (mnew > M) {
        const float corr = fast_exp2((M - mnew) * c2);   // 0 on the first pair (M = -inf)
        den *= corr;
#pragma unroll
        for (int e = 0; e < 32; ++e) acc[e] *= corr;
        M = mnew;
      }
      if (e0) {
        const float f = fast_exp2((m0.x - M) * c2);
        den = fmaf(f, m0.y, den);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          acc[4 * e] = fmaf(f, x0[e].x, acc[4 * e]);
          acc[4 * e + 1] = fmaf(f, x0[e].y, acc[4 * e + 1]);
          acc[4 * e + 2] = fmaf(f, x0[e].z, acc[4 * e + 2]);
          acc[4 * e + 3] = fmaf(f, x0[e].w, acc[4 * e + 3]);
        }
      }
      if (e1) {
        const float f = fast_exp2((m1.x - M) * c2);
        den = fmaf(f, m1.y, den);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          acc[4 * e] = fmaf(f, x1[e].x, acc[4 * e]);
          acc[4 * e + 1] = fmaf(f, x1[e].y, acc[4 * e + 1]);
          acc[4 * e + 2] = fmaf(f, x1[e].z, acc[4 * e + 2]);
          acc[4 * e + 3] = fmaf(f, x1[e].w, acc[4 * e + 3]);
        }
      }
    }
  }
  {
    const float inv = 1.0f / den;   // den >= 1: the partial holding M contributes f = 1 times its sum
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t hv[2], lv[2];
#pragma unroll
      for (int j = 0; j < 4; j += 2) {
        const float a = acc[4 * e + j] * inv, b = acc[4 * e + j + 1] * inv;
        hv[j >> 1] = pack_bf16x2(a, b);
        lv[j >> 1] = pack_bf16x2(a - bf16lo(hv[j >> 1]), b - bf16hi(hv[j >> 1]));
      }
      const int off = vl * kCmbLd + 64 * e + 4 * sub;
      *reinterpret_cast<uint2*>(ohi + off) = make_uint2(hv[0], hv[1]);
      *reinterpret_cast<uint2*>(olo + off) = make_uint2(lv[0], lv[1]);
    }
  }
  if (sub == 0) red[vl] = Mt;
  __syncthreads();
  if (tid == 0) {
    float mm = -INFINITY;
    for (int i = 0; i < kCmbV; ++i) mm = fmaxf(mm, red[i]);
    if (mm > -INFINITY) atomic_max_float(hmax + h, mm);   // approximate, raw; refined below
  }

  // ---- phase 2: O~^T = W_UV_h o_lat^T ----
  static_for<0, 2>([&](auto b) {
    static_for<kKs / 2, kKs>([&](auto kk) { wop[b][kk] = ldg16(wrow + b * 16 * kR + 32 * kk); });
  });
  f32x4 oc[2] = {f32x4{}, f32x4{}};
  static_for<0, kKs>([&](auto kk) {
    const int off = i16 * kCmbLd + 32 * kk + 8 * kq;
    const bf16x8 bh = as_bf16x8(*reinterpret_cast<const uint4*>(ohi + off));
    const bf16x8 bl = as_bf16x8(*reinterpret_cast<const uint4*>(olo + off));
    static_for<0, 2>([&](auto b) {
      oc[b] = mfma16(as_bf16x8(wop[b][kk]), bh, oc[b]);
      oc[b] = mfma16(as_bf16x8(wop[b][kk]), bl, oc[b]);
    });
  });
  const int64_t v = v0 + i16;
  if (v < bt) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const size_t idx = (static_cast<size_t>(v) * heads + h) * kV + 32 * wave + 16 * b + 4 * kq;
      float y[4] = {oc[b][0], oc[b][1], oc[b][2], oc[b][3]};
      if (gate) {
        const uint2 gv = *reinterpret_cast<const uint2*>(gate + idx);
        y[0] *= sigmoidf_(bf16lo(gv.x));
        y[1] *= sigmoidf_(bf16hi(gv.x));
        y[2] *= sigmoidf_(bf16lo(gv.y));
        y[3] *= sigmoidf_(bf16hi(gv.y));
      }
      if (OUT_BF16)
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + idx) =
            make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
      else
        *reinterpret_cast<float4*>(static_cast<float*>(out) + idx) = make_float4(y[0], y[1], y[2], y[3]);
    }
  }
}


// ---------------------------------------------------------------------------
// Max-logit refinement. The stream's logits use q_abs rounded to bf16, so
// the logit of row j carries an error of at most
//   delta_j = kDecErrCoef * max ||q_abs|| * ||row_j||
// (per tile, with the tile's largest row norm). The exact maximum E is then
// at least L = max over tiles of (streamed tile max - delta), and only a tile
// whose streamed max + delta reaches L can hold it. The split kernel keeps,
// per workgroup and head, its part of L and the tiles that pass against it;
// one workgroup per head here takes L over all split workgroups, keeps the
// listed tiles that still pass, and re-scores their rows in fp32 against
// q_abs carried to about 16 significant bits (its bf16 value plus the bf16
// rounding residual). The head's max logit is the maximum of those scores.
// If a list overflowed (near-ties: q = 0, repeated rows) the streamed maximum
// M is folded in as well, which is within max_j delta_j of E.
// ---------------------------------------------------------------------------
constexpr int kRefTiles = 128;   // candidate tiles per refine workgroup
constexpr int kRefSplit = 4;     // refine workgroups per head

// Grid (heads, kRefSplit): workgroup (h, y) takes the lists of the split
// workgroups w with w % kRefSplit == y. Scoring: one wave per listed tile;
// lane l takes row l % 32, half l / 32 of its 72 16-byte chunks.
__global__ void __launch_bounds__(256) absorbed_refine_kernel(
    int heads, const float* __restrict__ dlb, const int32_t* __restrict__ dcnt, const int4* __restrict__ dent,
    const float* __restrict__ hmax, const uint16_t* __restrict__ qabs, const uint16_t* __restrict__ qlo,
    const uint16_t* __restrict__ cache, int64_t cap, int tq, float scale, float* __restrict__ max_logit) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  __shared__ i32x4 tl[kRefTiles + 1];
  __shared__ float red[4];
  __shared__ int ntile, overflow;
  __shared__ __align__(16) float qe[4][kW];
  const int h = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float M = hmax[h];
  if (tid == 0) {
    ntile = 0;
    overflow = 0;
  }
  // ---- L over all split workgroups (kDecSplits == 256 threads)
  {
    const float lbw = wave_max(dlb[static_cast<size_t>(tid) * heads + h]);
    if (lane == 0) red[wave] = lbw;
  }
  // this thread's share of the lists: workgroup w, entries k = j (mod 4)
  const int w = kRefSplit * (tid >> 2) + blockIdx.y, j = tid & 3;
  const bool own = w < kDecSplits;
  const size_t o = static_cast<size_t>(own ? w : 0) * heads + h;
  const int c = own ? dcnt[o] : 0;
  i32x4 e[kDecList / 4];
  const i32x4* ent = reinterpret_cast<const i32x4*>(dent) + o * kDecList;
  // all slots, in flight with the count (slots past the count are ignored)
#pragma unroll
  for (int u = 0; u < kDecList / 4; ++u) e[u] = ent[j + 4 * u];
  __syncthreads();
  const float L = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  if (c > kDecList && j == 0) overflow = 1;
  // ---- the listed tiles that pass against L: slots reserved with one
  // atomic per thread, entries written without branches (an entry that does
  // not pass, or finds the list full, goes to the spare slot kRefTiles)
  {
    int npass = 0;
#pragma unroll
    for (int u = 0; u < kDecList / 4; ++u) {
      const int k = j + 4 * u;
      npass += (k < c && k < kDecList && __int_as_float(e[u][3]) >= L) ? 1 : 0;
    }
    int q = npass ? atomicAdd(&ntile, npass) : 0;
#pragma unroll
    for (int u = 0; u < kDecList / 4; ++u) {
      const int k = j + 4 * u;
      const bool p = k < c && k < kDecList && __int_as_float(e[u][3]) >= L;
      tl[p && q < kRefTiles ? q : kRefTiles] = e[u];
      q += p ? 1 : 0;
    }
    if (q > kRefTiles) overflow = 1;
  }
  __syncthreads();
  if (tid == 0 && overflow) atomic_max_float(max_logit + h, M * scale);   // some list overflowed
  // ---- rows of the listed tiles, one wave per tile
  const int nt = min(ntile, kRefTiles);
  float best = -INFINITY;
  float* q = qe[wave];
  const int rw = lane & 31, half = lane >> 5;
  for (int k = wave; k < nt; k += 4) {
    const i32x4 ti = tl[k];
    const int vs = ti[0], row0 = ti[1], nrows = ti[2];
    const uint16_t* qa = qabs + (static_cast<size_t>(vs) * heads + h) * kW;
    const uint16_t* ql = qlo + (static_cast<size_t>(vs) * heads + h) * kR;
    float qv[kW / 64];
#pragma unroll
    for (int u = 0; u < kW / 64; ++u) {
      const int c = lane + 64 * u;
      qv[u] = bf16_to_f32(qa[c]) + (c < kR ? bf16_to_f32(ql[c]) : 0.0f);
    }
    const bool rvalid = rw < nrows;
    const uint4* row = reinterpret_cast<const uint4*>(
        cache + (static_cast<size_t>(vs / tq) * cap + row0 + (rvalid ? rw : 0)) * kW) + (kChunks / 2) * half;
    // the lane's 36 chunks, all in flight together with the query
    uint4 rv[kChunks / 2];
#pragma unroll
    for (int u = 0; u < kChunks / 2; ++u) rv[u] = row[u];
#pragma unroll
    for (int u = 0; u < kW / 64; ++u) q[lane + 64 * u] = qv[u];
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    float sc = 0.0f;
    const float* qq = q + 8 * (kChunks / 2) * half;
#pragma unroll
    for (int u = 0; u < kChunks / 2; ++u) {
      const uint32_t* w4 = &rv[u].x;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sc = fmaf(qq[8 * u + 2 * e], bf16lo(w4[e]), fmaf(qq[8 * u + 2 * e + 1], bf16hi(w4[e]), sc));
    }
    sc += __shfl_xor(sc, 32, 64);
    if (rvalid) best = fmaxf(best, sc);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  }
  best = wave_max(best);
  if (lane == 0 && best > -INFINITY) atomic_max_float(max_logit + h, best * scale);
}

hipError_t launch_absorbed_bf16(int heads, float scale, bool out_bf16, const void* q, const void* cache,
                                int64_t cap, const int32_t* lens, int batch, int tq, const void* w_kv_b,
                                const void* gate, void* out, float* max_logit, bool init_max_logit, void* ws,
                                hipStream_t st, const QNorm& qn) {
  const AbsorbedWs L = absorbed_ws_layout(heads, batch, tq);
  char* base = static_cast<char*>(ws);
  float* dlb = reinterpret_cast<float*>(base + L.dlb);
  int32_t* dcnt = reinterpret_cast<int32_t*>(base + L.dcnt);
  int4* dent = reinterpret_cast<int4*>(base + L.dent);
  float* qn2 = reinterpret_cast<float*>(base + L.qn2);
  float* hmax = reinterpret_cast<float*>(base + L.hmax);
  uint16_t* qlo = reinterpret_cast<uint16_t*>(base + L.qlo);
  uint16_t* qabs = reinterpret_cast<uint16_t*>(base + L.qabs);
  int64_t* P = reinterpret_cast<int64_t*>(base + L.prefix);
  float* part_o = reinterpret_cast<float*>(base + L.part_o);
  float* part_ml = reinterpret_cast<float*>(base + L.part_ml);
  const int64_t bt = static_cast<int64_t>(batch) * tq;

  int32_t* nflag = reinterpret_cast<int32_t*>(base + L.nflag);
  hipError_t e;
  {
    TimedScope ts_("absorb_q", st);
    hipLaunchKernelGGL(absorb_q_kernel, dim3(heads, kR / 128), dim3(256), 0, st, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(w_kv_b), static_cast<int>(bt), heads, qabs, lens, tq, P, nflag,
                       init_max_logit ? max_logit : nullptr, qn2, hmax, qlo, qn.on ? 1 : 0,
                       static_cast<const uint16_t*>(qn.w), qn.eps);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    TimedScope ts_("absorbed_split", st);
    hipLaunchKernelGGL(absorbed_split_kernel, dim3(kDecSplits, (heads + kDecHeadsPerWg - 1) / kDecHeadsPerWg), dim3(256), 0, st,
                       static_cast<const uint16_t*>(cache), cap, tq, heads, bt, P, qabs, scale, part_o, part_ml,
                       nflag, qn2, dlb, dcnt, dent);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    TimedScope ts_("absorbed_fixup", st);
    hipLaunchKernelGGL(absorbed_fixup_kernel, dim3(kDecSplits), dim3(256), 0, st,
                       static_cast<const uint16_t*>(cache), cap, tq, heads, bt, kDecSplits, P, qabs, scale, part_o,
                       part_ml, nflag);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 cg(heads, static_cast<unsigned>((bt + kCmbV - 1) / kCmbV));
  if (out_bf16) {
    {
      TimedScope ts_("absorbed_combine", st);
      hipLaunchKernelGGL(absorbed_combine_kernel<true>, cg, dim3(256), 0, st, P, bt, heads, scale,
                         part_o, part_ml, static_cast<const uint16_t*>(w_kv_b),
                         static_cast<const uint16_t*>(gate), out, hmax);
    }
  } else {
    {
      TimedScope ts_("absorbed_combine", st);
      hipLaunchKernelGGL(absorbed_combine_kernel<false>, cg, dim3(256), 0, st, P, bt, heads, scale,
                         part_o, part_ml, static_cast<const uint16_t*>(w_kv_b),
                         static_cast<const uint16_t*>(gate), out, hmax);
    }
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    TimedScope ts_("absorbed_refine", st);
    hipLaunchKernelGGL(absorbed_refine_kernel, dim3(heads, kRefSplit), dim3(256), 0, st, heads, dlb, dcnt, dent,
                       hmax, qabs, qlo, static_cast<const uint16_t*>(cache), cap, tq, scale, max_logit);
  }
  return hipGetLastError();
}

}  // namespace mla
