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
// sequences' visible rows: the G workgroups own consecutive row ranges of
// equal cost, where a range's cost is its rows plus kSegCost rows for every
// sequence start inside it (starting a sequence reloads its queries and
// writes a partial), so every workgroup does the same work whatever the
// length mix. For every (workgroup, sequence) overlap it writes a partial
// (row max, denominator, unnormalised o_lat) for all heads; the combine
// kernel merges them by log-sum-exp.
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

// Row boundaries of the split workgroups, S[w] for w = 0 .. kDecSplits,
// stored right after P (S = P + bt + 1). The bt virtual sequences are laid
// end to end with kSegCost virtual rows before every one but the first (the
// cost of starting a sequence, in rows); workgroup w takes the cost interval
// [C w / G, C (w + 1) / G) of the total cost C, and a boundary that falls
// into such a gap snaps to the sequence start. Called by one workgroup after
// P is complete.
constexpr int64_t kSegCost = 256;
__device__ void absorbed_split_table(int64_t* __restrict__ P, int64_t bt) {
  int64_t* S = P + bt + 1;
  const int64_t C = P[bt] + kSegCost * (bt - 1);
  for (int w = threadIdx.x; w <= kDecSplits; w += blockDim.x) {
    const int64_t c = C * w / kDecSplits;
    // the last sequence v whose cost start P[v] + kSegCost v is at most c
    int64_t lo = 0, hi = bt - 1;
    while (lo < hi) {
      const int64_t mid = (lo + hi + 1) >> 1;
      if (P[mid] + kSegCost * mid <= c) lo = mid; else hi = mid - 1;
    }
    S[w] = P[lo] + min(c - (P[lo] + kSegCost * lo), P[lo + 1] - P[lo]);
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
                                                       uint16_t* __restrict__ qlo,
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
    __syncthreads();   // P is complete
    absorbed_split_table(P, bt);
    // max-logit slots start at -inf unless the caller accumulates into them
    if (ml_init && tid < heads) ml_init[tid] = -INFINITY;
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
// Split kernel. One workgroup of 8 waves per CU, two waves per SIMD (waves w
// and w + 4 share a SIMD). The workgroup's rows are visited in tiles of 32
// rows, segment (virtual sequence) by segment, as a software pipeline with
// one phase per tile and one barrier per phase:
//  - S waves 0-2, one per block of 32 heads, keep their heads' q_abs as MFMA
//    operands in registers. In phase i each forms S^T = C Q^T of tile i (36
//    MFMAs, each lane owns one head column, rows of C read as b128), the
//    tile's softmax weights against the segment's reference max, and writes
//    them to LDS in the MFMA B-operand order.
//  - PV waves 3-7 hold the latent accumulators O_lat^T = C^T P^T for a share
//    of the 48 (head block, 32 latent columns) blocks: waves 3 and 7 (which
//    share SIMD 3) 12 blocks each, waves 5 and 6 (beside S waves 1 and 2) 11
//    each, wave 4 (beside S wave 0, and keeping the max-logit candidate
//    lists) 2. In phase i they accumulate tile i-1 with the weights written
//    in phase i-1, C^T read through the LDS transpose read.
//  - The PV waves also stream the tiles into a ring of kStages LDS stages:
//    in phase i they issue the 37 wave-wide 1 KB copies of tile i+2 (waves
//    3-7: 10, 9, 6, 9 and 3 of them; buffer loads straight into LDS; the
//    buffer ends at the tile's last row, so reads past it return zeros) and
//    before the barrier each waits for its copies of tile i+1. A stage is
//    refilled two phases after its tile's S phase, once the PV phase of that
//    tile has ended.
// LDS tile layout: [32 rows][73 chunks of 8 bf16] (72 data chunks and one
// pad chunk per row, so rows are 36 banks apart and both read patterns are
// free of bank conflicts). A wave-wide copy fills 64 consecutive chunk
// slots. The pad slots of a stage's rows carry the S waves' partial squared
// row norms of that tile (the error bound of the max-logit refinement): S
// wave j sums the chunks 2 kk + g with kk = j (mod 3) it reads anyway, so
// the three partials cover each row once.
// The softmax takes every probability against a fixed reference, the first
// tile's max of the segment, so the accumulators are never rescaled; a head
// whose later logits exceed the reference by more than 64 in exp2 units is
// flagged (and counted in nflag) and its segment is recomputed by the fix-up
// kernel.
// Partials per (workgroup, virtual sequence) slot and head:
//   part_o[slot][h][r] = sum_j p_j c_j[r] (relative to the reference max),
//   part_ml[slot][h] = {reference max (raw), denominator, 0, flag}.
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
constexpr int kStages = 4;
constexpr int kSplitThreads = 512;
// Copies kc of a tile issued by each wave (first, count), weighted against
// the wave's other work: none for the S waves, 10, 9, 6, 9 and 3 for the PV
// waves 3-7.
constexpr int kCopyFirst[8] = {0, 0, 0, 9, 0, 19, 25, 34};
constexpr int kCopyCount[8] = {0, 0, 0, 10, 9, 6, 9, 3};
constexpr int kPBytes = 2 * 3 * 2 * 64 * 16;          // weights: 2 buffers x 3 head blocks x 2 halves x 64 lanes
static_assert(kCopyFirst[4] == 0 && kCopyFirst[3] == kCopyCount[4] && kCopyFirst[5] == kCopyFirst[3] + kCopyCount[3] &&
                  kCopyFirst[6] == kCopyFirst[5] + kCopyCount[5] && kCopyFirst[7] == kCopyFirst[6] + kCopyCount[6] &&
                  kCopyFirst[7] + kCopyCount[7] == kDmaCopies,
              "the waves' copies cover the tile once");
// Past the tile's slots a stage has room for the S waves' tile maxima (one
// float per head of the workgroup).
constexpr int kMaxOff = 16 * kTileSlots;
static_assert(kMaxOff + 4 * kDecHeadsPerWg <= kTileBytes, "tile maxima in the stage");
static_assert(kStages * kTileBytes + kPBytes <= 160 * 1024, "LDS of one workgroup");
static_assert(kDecHeadsPerWg == 96 && kDecRows == 32, "three head blocks of 32, tiles of 32 rows");

// Walk over a workgroup's row range [lo, lo + n), tile by tile and segment
// (virtual sequence) by segment. Positions are row offsets from lo, 32-bit (a
// range holds about total / G rows); the 64-bit prefix P is turned into offsets
// with 32-bit compares only. (This compiler has been seen to drop the
// VCC-to-SCC step of a 64-bit scalar select in this kernel, which made a
// cursor skip to its segment end; 32-bit scalar compares set SCC directly.)
struct TileCursor {
  int64_t lo;   // global index of the workgroup's first row
  int64_t vs;   // virtual sequence of the current tile
  int pos;      // offset of the current tile
  int seg_end;  // offset of the end of the current segment (at most n)
  int n;        // rows of the workgroup
};

// p - lo, for p > lo, as an offset clamped to n.
__device__ __forceinline__ int row_offset(int64_t p, int64_t lo, int n) {
  const uint64_t d = static_cast<uint64_t>(p - lo);
  uint32_t dh = static_cast<uint32_t>(d >> 32), dl = static_cast<uint32_t>(d);
  asm volatile("" : "+s"(dh), "+s"(dl));   // keeps the compares below 32-bit
  return (dh != 0u || dl > static_cast<uint32_t>(n)) ? n : static_cast<int>(dl);
}
// p <= lo (both row indices), with a 32-bit compare of the difference's high word.
__device__ __forceinline__ bool row_le(int64_t p, int64_t lo) {
  int h = static_cast<int>((lo - p) >> 32);
  asm volatile("" : "+s"(h));
  return h >= 0;
}

__device__ __forceinline__ void cursor_init(TileCursor& c, const int64_t* P, int64_t bt, int64_t lo, int64_t hi) {
  int vlo = 0, vhi = static_cast<int>(bt) - 1;
  while (vlo < vhi) {
    const int mid = (vlo + vhi + 1) >> 1;
    if (row_le(P[mid], lo)) vlo = mid; else vhi = mid - 1;
  }
  while (row_le(P[vlo + 1], lo)) ++vlo;
  c.lo = lo;
  c.vs = vlo;
  c.pos = 0;
  c.n = static_cast<int>(hi - lo);
  c.seg_end = row_offset(P[vlo + 1], lo, c.n);
}
__device__ __forceinline__ void cursor_next(TileCursor& c, const int64_t* P) {
  c.pos = min(c.pos + kDecRows, c.seg_end);
  if (c.pos >= c.seg_end && c.pos < c.n) {
    while (row_offset(P[c.vs + 1], c.lo, c.n) <= c.pos) ++c.vs;
    c.seg_end = row_offset(P[c.vs + 1], c.lo, c.n);
  }
}
__device__ __forceinline__ int cursor_rows(const TileCursor& c) { return min(kDecRows, c.seg_end - c.pos); }
// First row of the current tile within its virtual sequence.
__device__ __forceinline__ int64_t cursor_row0(const TileCursor& c, const int64_t* P) {
  return c.lo + c.pos - P[c.vs];
}

// Barrier without the fence __syncthreads carries (which would also wait for
// copies that are not needed yet); each wave waits for exactly what the
// others need first. The compiler keeps memory accesses on their side of it.
__device__ __forceinline__ void phase_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// The ring's stages and the softmax-weight buffers are LDS arrays of their own.
__shared__ __align__(16) char g_split_st0[kTileBytes];
__shared__ __align__(16) char g_split_st1[kTileBytes];
__shared__ __align__(16) char g_split_st2[kTileBytes];
__shared__ __align__(16) char g_split_st3[kTileBytes];
__shared__ __align__(16) uint4 g_split_p[kPBytes / 16];
template <int S>
__device__ __forceinline__ char* split_stage() {
  static_assert(S >= 0 && S < kStages, "stage");
  if constexpr (S == 0) return g_split_st0;
  else if constexpr (S == 1) return g_split_st1;
  else if constexpr (S == 2) return g_split_st2;
  else return g_split_st3;
}
__device__ __forceinline__ char* split_stage(int s) {
  return s == 0 ? g_split_st0 : s == 1 ? g_split_st1 : s == 2 ? g_split_st2 : g_split_st3;
}

// Buffer resource of the rows of one tile (4 dwords; reads past the last
// row return zeros).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 rows_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{static_cast<uint32_t>(a), static_cast<uint32_t>(a >> 32) & 0xffffu, bytes, 0x00020000u};
}
// 16 bytes per lane from the buffer at byte offset voff straight into LDS at
// lds + 16 lane (lds: an LDS address, the same for the whole wave). Written
// in asm: the compiler, which cannot tell the ring's stages apart behind a
// copy in flight, would otherwise wait for every copy before each LDS read;
// the callers order the copies against the reads with their own waits and
// barriers. M0 holds no compiler value in the code that issues them; the
// s_nop is the wait state an LDS-DMA load needs after a scalar write of M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // M0 is declared clobbered on purpose
__device__ __forceinline__ void dma16_rows(u32x4 rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc),
               "s"(lds)
               : "memory", "m0");
}
#pragma clang diagnostic pop
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)(p)));
}

// Issue this wave's copies of a tile (W: wave index): copy kc fills chunk
// slots 64 kc .. +63 of the stage (lane i: slot 64 kc + i = row r, chunk k of
// the tile).
template <int W>
__device__ __forceinline__ void split_copy(u32x4 rs, char* stage, int lane) {
  const uint32_t base = lds_addr(stage);
#pragma unroll
  for (int c = 0; c < kCopyCount[W]; ++c) {
    const int kc = kCopyFirst[W] + c;
    const int slot = 64 * kc + lane;
    const int r = slot / kRowSlots, k = slot - r * kRowSlots;
    dma16_rows(rs, static_cast<uint32_t>(r * (kW * 2) + 16 * k), base + 1024 * kc);
  }
}
__device__ __forceinline__ u32x4 tile_rsrc(const uint16_t* cache, int64_t cap, int tq, const int64_t* P,
                                          const TileCursor& c) {
  const int64_t b = c.vs / tq;
  const int64_t row0 = cursor_row0(c, P);
  return rows_rsrc(cache + (b * cap + row0) * kW, static_cast<uint32_t>(cursor_rows(c) * (kW * 2)));
}

// ---- S waves ----
struct SplitState {
  bf16x8 qf[kW / 16];
  float m_ref, l_part;
  bool overflow, first;
};

// Scores and softmax weights (pk: the B operands of the value product) for
// the tile at tb, and this wave's partial squared norm of the lane's row (the
// chunks 2 kk + g with kk = HB (mod 3), which it reads anyway; the three S
// waves' partials cover each row once). Returns the tile's approximate max
// logit of the lane's head.
template <int HB>
__device__ __forceinline__ float split_scores(const char* tb, int nrows, int lane, float c2, SplitState& S,
                                              uint32_t (&pk)[8], float& nsq) {
  const int g = lane >> 5;
  constexpr int kPf = 6;
  const uint4* arow = reinterpret_cast<const uint4*>(tb + 16 * ((lane & 31) * kRowSlots + g));
  uint4 af[kPf];
#pragma unroll
  for (int kk = 0; kk < kPf; ++kk) af[kk] = arow[2 * kk];
  // two accumulator chains (even and odd k-steps), added at the end
  f32x16 sacc = f32x16{}, sodd = f32x16{};
  float n = 0.0f;
#pragma unroll
  for (int kk = 0; kk < kW / 16; ++kk) {
    const uint4 u = af[kk % kPf];
    if (kk + kPf < kW / 16) af[kk % kPf] = arow[2 * (kk + kPf)];
    if (kk & 1) sodd = mfma32(as_bf16x8(u), S.qf[kk], sodd);
    else sacc = mfma32(as_bf16x8(u), S.qf[kk], sacc);
    if (kk % 3 == HB) {
      const bf16x8 v = as_bf16x8(u);
      n = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), __builtin_shufflevector(v, v, 0, 1), n, false);
      n = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), __builtin_shufflevector(v, v, 2, 3), n, false);
      n = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), __builtin_shufflevector(v, v, 4, 5), n, false);
      n = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), __builtin_shufflevector(v, v, 6, 7), n, false);
      asm volatile("" : "+v"(n));   // here, not sunk to the end of the loop (the chunk's registers are then free)
    }
  }
  nsq = n;
  // keep the reads kPf MFMAs ahead (the scheduler would otherwise sink them
  // next to their uses and expose the LDS latency on every MFMA)
  __builtin_amdgcn_sched_group_barrier(0x100, kPf, 0);
#pragma unroll
  for (int kk = 0; kk < kW / 16; ++kk) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (kk + kPf < kW / 16) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  sacc += sodd;
  if (nrows < kDecRows) {
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (acc_row(e, g) >= nrows) sacc[e] = -INFINITY;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < 16; e += 2) mx = fmax3_(mx, sacc[e], sacc[e + 1]);
  mx = xor32_max(mx);
  if (S.first) S.m_ref = mx;
  S.overflow = S.overflow || (mx - S.m_ref) * c2 > 64.0f;
  const float moff = -S.m_ref * c2;
  float psum = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; e += 2) {
    const float p0 = fast_exp2(fmaf(sacc[e], c2, moff));
    const float p1 = fast_exp2(fmaf(sacc[e + 1], c2, moff));
    psum += p0 + p1;
    pk[e >> 1] = pack_bf16x2(p0, p1);
  }
  S.l_part += psum;
  S.first = false;
  return mx;
}

// Maximum over the 32 lanes of each half of the wave (quad swaps, the 8- and
// 16-lane mirrors, then one exchange of 16-lane rows; no LDS traffic).
__device__ __forceinline__ float half_max32(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(v, fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}

// Candidate list of one head in one split workgroup: the slots dent[o][.] of
// the workgroup, kept by the lane that owns the head (count and bound in its
// registers). lb is a lower bound of the head's exact max logit (the largest
// tile max minus its error bound so far); a tile can hold the exact maximum
// only if its max plus its error bound reaches lb, so entries below the
// current lb are dropped whenever the list fills up. cnt == kDecList + 1
// marks a list that overflowed with live entries. Entries: {virtual
// sequence, first row, rows, bits of the upper bound}.
__device__ __forceinline__ void cand_compact(int4* list, int& cnt, float lb) {
  __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0): the lane's earlier stores to the list are done
  int j = 0;
  for (int k = 0; k < cnt; ++k) {
    int4 e;
    e.x = __hip_atomic_load(&list[k].x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    e.y = __hip_atomic_load(&list[k].y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    e.z = __hip_atomic_load(&list[k].z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    e.w = __hip_atomic_load(&list[k].w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__int_as_float(e.w) >= lb) list[j++] = e;
  }
  cnt = j;
}
__device__ __forceinline__ void cand_record(int4* list, int& cnt, float& lb, float mx, float d, int vs, int row0,
                                            int nrows) {
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
  list[cnt++] = make_int4(vs, row0, nrows, __float_as_int(u));
}

template <int HB>
__device__ __forceinline__ void split_s_wave(int ntiles, int lane, int64_t lo, int64_t hi, int heads, int64_t bt,
                                             const int64_t* P, const uint16_t* cache, int64_t cap, int tq,
                                             const uint16_t* qabs, float c2, float* part_ml, int32_t* nflag) {
  const int g = lane >> 5, l32 = lane & 31;
  const int head = 32 * (3 * static_cast<int>(blockIdx.y) + HB) + l32;
  const bool hvalid = head < heads;
  const int hq = hvalid ? head : 0;
  static_assert(kCopyCount[HB] == 0, "the S waves issue no copies");
  TileCursor cur;   // the tile being scored
  cursor_init(cur, P, bt, lo, hi);
  phase_barrier();   // tile 0 has landed
  SplitState S;
  bool seg_new = true;
  for (int i = 0; i <= ntiles; ++i) {
    if (i < ntiles) {
      const int64_t vs = cur.vs;
      if (seg_new) {
        const uint16_t* qrow = qabs + (static_cast<size_t>(vs) * heads + hq) * kW + 8 * g;
#pragma unroll
        for (int kk = 0; kk < kW / 16; ++kk)
          S.qf[kk] = as_bf16x8(hvalid ? ldg16(qrow + 16 * kk) : make_uint4(0, 0, 0, 0));
        // Fixed reference max per segment (the first tile's): probabilities
        // relative to it may exceed 1 but stay far inside the bf16 / fp32
        // range unless a later logit exceeds it by more than 64 / c2 (p >
        // 2^64; flagged, and such segments are recomputed by the fix-up
        // kernel).
        S.m_ref = 0.0f;
        S.l_part = 0.0f;
        S.overflow = false;
        S.first = true;
        seg_new = false;
      }
      char* tb = split_stage(i % kStages);
      uint32_t pk[8];
      float nsq;
      const float mx = split_scores<HB>(tb, cursor_rows(cur), lane, c2, S, pk, nsq);
      // weights in the value product's B-operand order; for the candidate
      // record made in the next phase, the norm partial of row l32 in its
      // pad slot (float HB) and the tile max of each head past the tile
      uint4* pw = g_split_p + ((i & 1) * 3 + HB) * 128;
      pw[lane] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      pw[64 + lane] = make_uint4(pk[4], pk[5], pk[6], pk[7]);
      nsq = xor32_sum(nsq);
      if (g == 0) {
        *reinterpret_cast<float*>(tb + 16 * (l32 * kRowSlots + kChunks) + 4 * HB) = nsq;
        *reinterpret_cast<float*>(tb + kMaxOff + 4 * (32 * HB + l32)) = mx;
      }
      cursor_next(cur, P);
      if (cur.pos >= cur.seg_end || cur.vs != vs) {
        // the segment ends with this tile: its softmax statistics
        if (hvalid) {
          const size_t slot = static_cast<size_t>(blockIdx.x) + static_cast<size_t>(vs);
          const float l_tot = xor32_sum(S.l_part);
          if (g == 0)
            *reinterpret_cast<float4*>(part_ml + (slot * heads + head) * 4) =
                make_float4(S.m_ref, l_tot, 0.0f, S.overflow ? 1.0f : 0.0f);
        }
        if (__ballot(hvalid && S.overflow) && lane == 0) atomicAdd(nflag, 1);
        seg_new = true;
      }
    }
    wait_lgkm0();
    phase_barrier();
  }
}

// ---- PV waves ----
// Blocks B0 .. B0+NB-1 of the 48 (block b: head block b / 16, latent columns
// 32 (b % 16) .. +31), at most two head blocks.
template <int B0, int NB>
__device__ __forceinline__ void split_pv(const char* tb, const uint4* pb, int lane, f32x16 (&o)[12]) {
  constexpr int H0 = B0 / 16;
  constexpr int N0 = (NB < 16 - B0 % 16) ? NB : 16 - B0 % 16;   // blocks in head block H0
  const int i16 = lane & 15;
  const int mhalf = 16 * ((lane >> 4) & 1);
  const int g = lane >> 5;
  bf16x8 p0[2], p1[2];
  p0[0] = as_bf16x8(pb[H0 * 128 + lane]);
  p0[1] = as_bf16x8(pb[H0 * 128 + 64 + lane]);
  if constexpr (N0 < NB) {
    p1[0] = as_bf16x8(pb[(H0 + 1) * 128 + lane]);
    p1[1] = as_bf16x8(pb[(H0 + 1) * 128 + 64 + lane]);
  }
  const lds_u16* tl = (const lds_u16*)(tb);
  const lds_u16* rowp = tl + (4 * g + (i16 >> 2)) * (8 * kRowSlots) + mhalf + 4 * (i16 & 3);
  // MFMA m = NB ks + j: k-step ks (rows 16 ks .. +15) of block j
  auto ptr = [&](int m) {
    const int ks = m / NB, cb = (B0 + m % NB) % 16;
    return rowp + ks * 16 * (8 * kRowSlots) + 32 * cb;
  };
  constexpr int kPv = NB > 8 ? 3 : 4;   // operand reads in flight (registers are tight at 12 blocks)
  v4s t0[kPv], t1[kPv];
#pragma unroll
  for (int m = 0; m < kPv; ++m) {
    t0[m] = lds_tr4(ptr(m));
    t1[m] = lds_tr4(ptr(m) + 8 * (8 * kRowSlots));
  }
#pragma unroll
  for (int m = 0; m < 2 * NB; ++m) {
    const bf16x8 a = cat_bf16(t0[m % kPv], t1[m % kPv]);
    if (m + kPv < 2 * NB) {
      t0[m % kPv] = lds_tr4(ptr(m + kPv));
      t1[m % kPv] = lds_tr4(ptr(m + kPv) + 8 * (8 * kRowSlots));
    }
    const int ks = m / NB, j = m % NB;
    o[j] = mfma32(a, j < N0 ? (ks ? p0[1] : p0[0]) : (ks ? p1[1] : p1[0]), o[j]);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * kPv, 0);
#pragma unroll
  for (int m = 0; m < 2 * NB; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
}

// PV wave with blocks B0 .. B0+NB-1 of the value product. The wave with CAND
// also keeps the max-logit candidate lists of the workgroup's 96 heads (lane
// l < 32 owns head l of each head block): for the tile accumulated in a
// phase, the tile's largest row norm (from the S waves' partials in the
// stage's pad slots) and the tile max of each head (past the tile's slots)
// give the tile's error bound and its entry.
template <int W, int B0, int NB, bool CAND>
__device__ __forceinline__ void split_pv_wave(int ntiles, int lane, int64_t lo, int64_t hi, int heads, int64_t bt,
                                              const int64_t* P, const uint16_t* cache, int64_t cap, int tq,
                                              float* part_o, const float* qn2, float* dlb, int32_t* dcnt,
                                              int4* dent) {
  constexpr int NC = kCopyCount[W];
  const int g = lane >> 5, l32 = lane & 31;
  float qerr[3], clb[3];
  int ccnt[3];
  int4* clst[3];
  bool cvalid[3];
  size_t co[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int chead = 32 * (3 * static_cast<int>(blockIdx.y) + k) + l32;
    cvalid[k] = CAND && chead < heads;
    const int cq = cvalid[k] ? chead : 0;
    qerr[k] = CAND ? kDecErrCoef * sqrtf((qn2[4 * cq] + qn2[4 * cq + 1]) + (qn2[4 * cq + 2] + qn2[4 * cq + 3]))
                   : 0.0f;
    co[k] = static_cast<size_t>(blockIdx.x) * heads + cq;
    clst[k] = dent + co[k] * kDecList;
    clb[k] = -INFINITY;
    ccnt[k] = 0;
  }
  TileCursor pc, lc;   // the tile being accumulated, the tile being loaded
  cursor_init(pc, P, bt, lo, hi);
  cursor_init(lc, P, bt, lo, hi);
  if constexpr (NC > 0) {
    // this wave's copies of tiles 0 and 1
    split_copy<W>(tile_rsrc(cache, cap, tq, P, lc), split_stage(0), lane);
    cursor_next(lc, P);
    if (ntiles > 1) {
      split_copy<W>(tile_rsrc(cache, cap, tq, P, lc), split_stage(1), lane);
      cursor_next(lc, P);
      wait_vmcnt<NC>();
    } else {
      wait_vmcnt<0>();
    }
  }
  phase_barrier();   // tile 0 has landed
  f32x16 o[12];
#pragma unroll
  for (int j = 0; j < 12; ++j) o[j] = f32x16{};
  for (int i = 0; i <= ntiles; ++i) {
    const bool load = NC > 0 && i + 2 < ntiles;
    if (load) {
      split_copy<W>(tile_rsrc(cache, cap, tq, P, lc), split_stage((i + 2) % kStages), lane);
      cursor_next(lc, P);
    }
    if (i >= 1) {
      // tile i-1, with the weights the S waves wrote in the previous phase
      const int t = i - 1;
      const char* tb = split_stage(t % kStages);
      split_pv<B0, NB>(tb, g_split_p + (t & 1) * 3 * 128, lane, o);
      const int64_t vs = pc.vs;
      if constexpr (CAND) {
        // the tile's largest row norm from the S waves' partials
        const int nrows = cursor_rows(pc);
        const float* pad = reinterpret_cast<const float*>(tb + 16 * (l32 * kRowSlots + kChunks));
        const float tn = sqrtf(half_max32(l32 < nrows ? (pad[0] + pad[1]) + pad[2] : 0.0f));
        const float* tmax = reinterpret_cast<const float*>(tb + kMaxOff);
        const int row0 = static_cast<int>(cursor_row0(pc, P));
#pragma unroll
        for (int k = 0; k < 3; ++k)
          if (cvalid[k] && g == 0)
            cand_record(clst[k], ccnt[k], clb[k], tmax[32 * k + l32], qerr[k] * tn, static_cast<int>(vs), row0, nrows);
      }
      cursor_next(pc, P);
      if (pc.pos >= pc.seg_end || pc.vs != vs) {
        // the segment ends with this tile: this wave's blocks of its partial
        const size_t slot = static_cast<size_t>(blockIdx.x) + static_cast<size_t>(vs);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int b = B0 + j;
          const int head = 32 * (3 * static_cast<int>(blockIdx.y) + b / 16) + l32;
          if (head < heads) {
            float* po = part_o + (slot * heads + head) * kR + 32 * (b % 16);
#pragma unroll
            for (int grp = 0; grp < 4; ++grp)
              *reinterpret_cast<float4*>(po + 8 * grp + 4 * g) =
                  make_float4(o[j][4 * grp], o[j][4 * grp + 1], o[j][4 * grp + 2], o[j][4 * grp + 3]);
          }
          o[j] = f32x16{};
        }
      }
    }
    if constexpr (NC > 0) {
      if (load) wait_vmcnt<NC>(); else wait_vmcnt<0>();
    }
    wait_lgkm0();
    phase_barrier();
  }
  // the heads' bounds and live candidates of this workgroup
  if constexpr (CAND) {
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      if (cvalid[k] && g == 0) {
        if (ccnt[k] <= kDecList) cand_compact(clst[k], ccnt[k], clb[k]);
        dlb[co[k]] = clb[k];
        dcnt[co[k]] = ccnt[k];
      }
    }
  }
}

__global__ void __launch_bounds__(kSplitThreads) absorbed_split_kernel(
    const uint16_t* __restrict__ cache, int64_t cap, int tq, int heads, int64_t bt,
    const int64_t* __restrict__ P, const uint16_t* __restrict__ qabs, float scale,
    float* __restrict__ part_o, float* __restrict__ part_ml, int32_t* __restrict__ nflag,
    const float* __restrict__ qn2, float* __restrict__ dlb, int32_t* __restrict__ dcnt, int4* __restrict__ dent) {

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t* S = P + bt + 1;   // the workgroups' row boundaries
  const int64_t lo = S[blockIdx.x], hi = S[blockIdx.x + 1];
  if (lo >= hi) {
    // no rows: no bound and no candidates for this workgroup's heads
    for (int h = 96 * static_cast<int>(blockIdx.y) + tid; h < min(heads, 96 * (static_cast<int>(blockIdx.y) + 1));
         h += kSplitThreads) {
      dlb[blockIdx.x * heads + h] = -INFINITY;
      dcnt[blockIdx.x * heads + h] = 0;
    }
    return;
  }
  int ntiles = 0;
  {
    TileCursor c;
    cursor_init(c, P, bt, lo, hi);
    while (c.pos < c.n) {
      ++ntiles;
      cursor_next(c, P);
    }
  }
  const float c2 = scale * kLog2e;
  switch (wave) {
    case 0:
      split_s_wave<0>(ntiles, lane, lo, hi, heads, bt, P, cache, cap, tq, qabs, c2, part_ml, nflag);
      break;
    case 1:
      split_s_wave<1>(ntiles, lane, lo, hi, heads, bt, P, cache, cap, tq, qabs, c2, part_ml, nflag);
      break;
    case 2:
      split_s_wave<2>(ntiles, lane, lo, hi, heads, bt, P, cache, cap, tq, qabs, c2, part_ml, nflag);
      break;
    // value-product blocks: 12 + 12 for the two waves of SIMD 3, 2 + 11 + 11
    // for the partners of the S waves (wave 4 also keeps the candidate lists)
    case 3:
      split_pv_wave<3, 0, 12, false>(ntiles, lane, lo, hi, heads, bt, P, cache, cap, tq, part_o, qn2, dlb, dcnt, dent);
      break;
    case 4:
      split_pv_wave<4, 24, 2, true>(ntiles, lane, lo, hi, heads, bt, P, cache, cap, tq, part_o, qn2, dlb, dcnt, dent);
      break;
    case 5:
      split_pv_wave<5, 26, 11, false>(ntiles, lane, lo, hi, heads, bt, P, cache, cap, tq, part_o, qn2, dlb, dcnt, dent);
      break;
    case 6:
      split_pv_wave<6, 37, 11, false>(ntiles, lane, lo, hi, heads, bt, P, cache, cap, tq, part_o, qn2, dlb, dcnt, dent);
      break;
    default:
      split_pv_wave<7, 12, 12, false>(ntiles, lane, lo, hi, heads, bt, P, cache, cap, tq, part_o, qn2, dlb, dcnt, dent);
      break;
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
    const uint16_t* __restrict__ cache, int64_t cap, int tq, int heads, int64_t bt,
    const int64_t* __restrict__ P, const uint16_t* __restrict__ qabs, float scale, float* __restrict__ part_o,
    float* __restrict__ part_ml, const int32_t* __restrict__ nflag) {
  if (*nflag == 0) return;   // nothing was flagged (the common case)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t* S = P + bt + 1;   // the split workgroups' row boundaries
  const int64_t lo = S[blockIdx.x], hi = S[blockIdx.x + 1];
  if (lo >= hi) return;
  const float c2 = scale * kLog2e;
  TileCursor cur;
  cursor_init(cur, P, bt, lo, hi);
  while (cur.pos < cur.n) {
    const int64_t vs = cur.vs;
    // the segment's rows within the sequence
    const int64_t seg_beg = cursor_row0(cur, P), seg_len = cur.seg_end - cur.pos;
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
      for (int64_t r = seg_beg; r < seg_beg + seg_len; ++r) {
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
        ml[3] = 0.0f;
      }
    }
    cur.pos = cur.seg_end;
    if (cur.pos < cur.n) {
      while (row_offset(P[cur.vs + 1], cur.lo, cur.n) <= cur.pos) ++cur.vs;
      cur.seg_end = row_offset(P[cur.vs + 1], cur.lo, cur.n);
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

// The split workgroup whose rows contain `row`: the largest w with S[w] <=
// row (S: the split kernel's row boundaries; empty workgroups share their
// boundary with the next one).
__device__ __forceinline__ int split_of_row(const int64_t* S, int64_t row) {
  int lo = 0, hi = kDecSplits - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (S[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ float group16_max(float v) {
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

template <bool OUT_BF16>
__device__ __forceinline__ void absorbed_combine_body(
    int hblk, int yblk, const int64_t* __restrict__ P, int64_t bt, int heads, float scale, const float* __restrict__ part_o,
    const float* __restrict__ part_ml, const uint16_t* __restrict__ w, const uint16_t* __restrict__ gate,
    void* __restrict__ out) {
  __shared__ __align__(16) uint16_t ohi[kCmbV * kCmbLd];
  __shared__ __align__(16) uint16_t olo[kCmbV * kCmbLd];
  const int h = hblk;
  const int64_t v0 = static_cast<int64_t>(yblk) * kCmbV;
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
  float den = 1.0f;
  if (vs < bt) {
    const int64_t* S = P + bt + 1;
    const int wa = split_of_row(S, P[vs]);
    const int wb = split_of_row(S, P[vs + 1] - 1);
    auto nonempty = [&](int s) { return S[s] < S[s + 1]; };
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
  __syncthreads();   // o_lat (hi, lo) of the workgroup's sequences is in LDS

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
// If a list overflowed (near-ties: q = 0, repeated rows), the refine
// workgroup re-scores instead, per split workgroup, every tile of its row
// range (its own list overflowed) or its listed tiles that pass against L,
// so the result is the same exact maximum, only slower to reach.
// ---------------------------------------------------------------------------
constexpr int kRefTiles = 128;   // candidate tiles per refine workgroup
constexpr int kRefSplit = 4;     // refine workgroups per head

// Grid (heads, kRefSplit): workgroup (h, y) takes the lists of the split
// workgroups w with w % kRefSplit == y. Scoring: one wave per tile; lane l
// takes row l % 32, half l / 32 of its 72 16-byte chunks. P (bt + 1 row
// offsets of the virtual sequences) gives the split workgroups' row ranges
// for the overflow path.
__device__ __forceinline__ void absorbed_refine_body(
    int hblk, int yblk, int heads, const float* __restrict__ dlb, const int32_t* __restrict__ dcnt, const int4* __restrict__ dent,
    const int64_t* __restrict__ P, int64_t bt, const uint16_t* __restrict__ qabs, const uint16_t* __restrict__ qlo,
    const uint16_t* __restrict__ cache, int64_t cap, int tq, float scale, float* __restrict__ max_logit) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  __shared__ i32x4 tl[kRefTiles + 1];
  __shared__ float red[4];
  __shared__ int ntile, overflow;
  __shared__ __align__(16) float qe[4][kW];
  const int h = hblk;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar row walk below)
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
  const int w = kRefSplit * (tid >> 2) + yblk, j = tid & 3;
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
  float best = -INFINITY;
  float* q = qe[wave];
  const int rw = lane & 31, half = lane >> 5;
  // the rows [row0, row0 + nrows) of virtual sequence vs, one per lane pair,
  // scored in fp32 against q_abs + residual; the maximum goes into best
  auto score_tile = [&](int vs, int row0, int nrows) {
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
  };
  if (!overflow) {
    // ---- the listed tiles that pass, one wave per tile
    const int nt = min(ntile, kRefTiles);
    for (int k = wave; k < nt; k += 4) {
      const i32x4 ti = tl[k];
      score_tile(ti[0], ti[1], ti[2]);
    }
  } else {
    // ---- a list overflowed: each wave takes every fourth of this
    // workgroup's split workgroups and scores all tiles of its row range
    // (walked as the split kernel walks it) when its own list overflowed,
    // else its listed tiles that pass against L
    const int64_t* S = P + bt + 1;
    for (int i = wave; kRefSplit * i + yblk < kDecSplits; i += 4) {
      const int ws = kRefSplit * i + yblk;
      const size_t os = static_cast<size_t>(ws) * heads + h;
      const int cs = dcnt[os];
      if (cs > kDecList) {
        const int64_t lo = S[ws], hi = S[ws + 1];
        if (lo >= hi) continue;
        TileCursor cur;
        cursor_init(cur, P, bt, lo, hi);
        while (cur.pos < cur.n) {
          score_tile(static_cast<int>(cur.vs), static_cast<int>(cursor_row0(cur, P)), cursor_rows(cur));
          cursor_next(cur, P);
        }
      } else {
        const i32x4* es = reinterpret_cast<const i32x4*>(dent) + os * kDecList;
        for (int k = 0; k < cs; ++k) {
          const i32x4 ti = es[k];
          if (__int_as_float(ti[3]) >= L) score_tile(ti[0], ti[1], ti[2]);
        }
      }
    }
  }
  best = wave_max(best);
  if (lane == 0 && best > -INFINITY) atomic_max_float(max_logit + h, best * scale);
}

// The combine and the max-logit refinement read disjoint inputs (partials
// against candidate lists) and write disjoint outputs, so they share one
// launch on a grid (heads, kRefSplit + blocks of kCmbV virtual sequences):
// rows y < kRefSplit refine (list share y), the rest combine (block
// y - kRefSplit). The dispatcher walks x fastest, so the refine workgroups go
// out first. Two waves per SIMD: the refine part alone would take 280
// registers (one wave per SIMD, which also halves the combine's occupancy);
// capped at 256 it spills 96 bytes per lane and the call is about 2 % faster.
template <bool OUT_BF16>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) absorbed_finish_kernel(
    int heads, const int64_t* __restrict__ P, int64_t bt, float scale, const float* __restrict__ part_o,
    const float* __restrict__ part_ml, const uint16_t* __restrict__ w, const uint16_t* __restrict__ gate,
    void* __restrict__ out, const float* __restrict__ dlb, const int32_t* __restrict__ dcnt,
    const int4* __restrict__ dent, const uint16_t* __restrict__ qabs, const uint16_t* __restrict__ qlo,
    const uint16_t* __restrict__ cache, int64_t cap, int tq, float* __restrict__ max_logit) {
  const int h = static_cast<int>(blockIdx.x);
  const int y = static_cast<int>(blockIdx.y);
  if (y < kRefSplit) {
    absorbed_refine_body(h, y, heads, dlb, dcnt, dent, P, bt, qabs, qlo, cache, cap, tq, scale, max_logit);
  } else {
    absorbed_combine_body<OUT_BF16>(h, y - kRefSplit, P, bt, heads, scale, part_o, part_ml, w, gate, out);
  }
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
                       init_max_logit ? max_logit : nullptr, qn2, qlo, qn.on ? 1 : 0,
                       static_cast<const uint16_t*>(qn.w), qn.eps);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    TimedScope ts_("absorbed_split", st);
    hipLaunchKernelGGL(absorbed_split_kernel, dim3(kDecSplits, (heads + kDecHeadsPerWg - 1) / kDecHeadsPerWg), dim3(kSplitThreads), 0, st,
                       static_cast<const uint16_t*>(cache), cap, tq, heads, bt, P, qabs, scale, part_o, part_ml,
                       nflag, qn2, dlb, dcnt, dent);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    TimedScope ts_("absorbed_fixup", st);
    hipLaunchKernelGGL(absorbed_fixup_kernel, dim3(kDecSplits), dim3(256), 0, st,
                       static_cast<const uint16_t*>(cache), cap, tq, heads, bt, P, qabs, scale, part_o,
                       part_ml, nflag);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 fg(heads, static_cast<unsigned>(kRefSplit + (bt + kCmbV - 1) / kCmbV));
  {
    TimedScope ts_("absorbed_finish", st);
    if (out_bf16)
      hipLaunchKernelGGL(absorbed_finish_kernel<true>, fg, dim3(256), 0, st, heads, P,
                         bt, scale, part_o, part_ml, static_cast<const uint16_t*>(w_kv_b),
                         static_cast<const uint16_t*>(gate), out, dlb, dcnt, dent, qabs, qlo,
                         static_cast<const uint16_t*>(cache), cap, tq, max_logit);
    else
      hipLaunchKernelGGL(absorbed_finish_kernel<false>, fg, dim3(256), 0, st, heads,
                         P, bt, scale, part_o, part_ml, static_cast<const uint16_t*>(w_kv_b),
                         static_cast<const uint16_t*>(gate), out, dlb, dcnt, dent, qabs, qlo,
                         static_cast<const uint16_t*>(cache), cap, tq, max_logit);
  }
  return hipGetLastError();
}

}  // namespace mla
