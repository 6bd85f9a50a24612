// Backward of the training-form prefill (bf16): the gradients of the
// equation list of "Kimi K3 · Gated MLA · OpenModelAtlas" (expansion
// [k^C v] = c^KV W_UKV, K_h = [K^C_h, k^S], S = Q K^T / sqrt(192), causal
// softmax, O~ = A V, o = sigma(g) . o~) with respect to q, c^KV, k^S,
// kv_b_proj.weight and the gate logits, for an upstream gradient dO of o:
//   dO~ = dO . sigma(g),  dg = dO . o . (1 - sigma(g)),  D = rowsum(dO . o),
//   P = exp(scale S - lse) (recomputed from the forward's LSE),
//   dV = P^T dO~,  dS' = P . (dO~ V^T - D),  dQ = scale dS' K,  dK = scale dS'^T Q,
// then [dK^C | dV] flows back through W_UKV into c^KV and the weight, and the
// k^S part of dK sums over the heads.
//
// No L x L plane is formed: the causal half of each head's score matrix is
// recomputed tile by tile on the matrix cores, twice.
//   dK/dV pass: one workgroup = one head x 128 keys of one sequence, 4 waves
//     of 32 keys; a wave keeps its keys' K and V fragments and its dK, dV
//     accumulators in registers and visits the query tiles (64 queries) from
//     the end of the sequence down to its diagonal:
//       S = Q K^T, dP = dO~ V^T (accumulator lane = key), P, dS';
//       dV += P^T dO~, dK += dS'^T Q: P and dS' leave the accumulators as the
//       key-major operand directly; dO~ and Q are read with the LDS transpose read.
//   dQ pass: one workgroup = one head x 128 queries, 4 waves of 32 queries
//     holding Q and dO~ fragments and the dQ accumulator; key tiles (64 keys)
//     from the start of the sequence up to the diagonal:
//       S^T = K Q^T, dP^T = V dO~^T (accumulator lane = query), dS';
//       dQ += dS' K (K by the transpose read).
// Both passes stream their tiles into two LDS stages with buffer loads
// straight to LDS, one tile ahead. Work items (sequence, 128-row block) are
// ordered longest first by a one-workgroup plan kernel that reads cu_seqlens
// on the device, so the whole backward is asynchronous on the stream.
// The expansion [K^C | V] = c^KV W_UKV^T-rows and the products
// dc^KV = [dK^C | dV] W_UKV, dW = [dK^C | dV]^T c^KV run on the NT GEMM kernel.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "mla_common.h"
#include "mla_internal.h"
#include "timing.h"

#pragma clang diagnostic ignored "-Winline-asm"

namespace mla {

namespace {

constexpr int kBwThreads = 256;   // 4 waves
constexpr int kBwBlock = 128;     // keys (dK/dV pass) or queries (dQ pass) per workgroup
constexpr int kBwTile = 64;       // queries (dK/dV pass) or keys (dQ pass) per inner tile

// LDS tiles of 64 rows in 16-byte units. A 128-feature region holds 16 units
// per row, unit u of row r at slot 16 r + (u ^ sw16(r)); a 64-feature region
// holds 8, unit u at slot 8 r + (u ^ sw8(r)). Both swizzles keep the two read
// patterns free of bank conflicts: 16 consecutive rows at one unit (operand
// rows, 16 lanes of a 16-byte read) and 4 consecutive rows from a multiple of
// 4 times an aligned quad of units (the transpose read).
__host__ __device__ constexpr int sw16(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__host__ __device__ constexpr int sw8(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }
constexpr int kReg16 = kBwTile * 16 * 16;   // 16 KB
constexpr int kReg8 = kBwTile * 8 * 16;     // 8 KB
// dK/dV pass stage: Q^C | Q^R | dO~ | {lse log2(e), D} of the 64 query rows (1 KB slot)
constexpr int kKvStage = 2 * kReg16 + kReg8 + 1024;
// dQ pass stage: K^C | k^S | V
constexpr int kQStage = 2 * kReg16 + kReg8;
static_assert(kKvStage % 1024 == 0 && kQStage % 1024 == 0, "stage offsets keep the swizzle bits clear");

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t lds_off(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_char*)(p)));
}

// Buffer resource over [base, base + bytes): loads past the end read zeros.
__device__ __forceinline__ u32x4 bw_rsrc(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t n = bytes <= 0 ? 0u : (bytes >= 0xffffffffLL ? 0xffffffffu : static_cast<uint32_t>(bytes));
  return u32x4{static_cast<uint32_t>(a), static_cast<uint32_t>(a >> 32) & 0xffffu, n, 0x00020000u};
}

// 16 bytes per lane from buffer offset voff straight into LDS at lds + 16 lane.
// Issued as inline assembly so that the compiler does not order its own LDS
// reads of the other stage behind these copies; the caller waits for them
// (vmcnt) before the barrier that publishes the stage. M0 is written here,
// and one wait state separates that write from the load that reads it.
__device__ __forceinline__ void bw_dma16(u32x4 rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc),
               "s"(lds)
               : "memory", "m0");
}

__device__ __forceinline__ void bw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Copies of one wave's share of a 64-row tile region (the region is split
// over the 4 waves in whole 1 KB copies: rows 16 w .. 16 w + 15).
//   16-unit region: copy i (0..3) holds rows 16 w + 4 i + lane / 16
//   8-unit region:  copy i (0..1) holds rows 16 w + 8 i + lane / 8
// rs: buffer over the region's rows (row stride rstride bytes), col: byte
// offset of the region's first feature within a row.
__device__ __forceinline__ void copy16(u32x4 rs, int64_t rstride, int col, uint32_t lds, int w, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * w + 4 * i + (lane >> 4);
    const int u = (lane & 15) ^ sw16(r);
    bw_dma16(rs, static_cast<uint32_t>(r * rstride + col + 16 * u), lds + (16 * 16) * (16 * w + 4 * i));
  }
}
__device__ __forceinline__ void copy8(u32x4 rs, int64_t rstride, int col, uint32_t lds, int w, int lane) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 16 * w + 8 * i + (lane >> 3);
    const int u = (lane & 7) ^ sw8(r);
    bw_dma16(rs, static_cast<uint32_t>(r * rstride + col + 16 * u), lds + (8 * 16) * (16 * w + 8 * i));
  }
}

// Per-lane LDS byte offsets of the two read patterns (lane l, half g = l / 32).
//   row16 / row8: operand row R0 + l % 32 (R0 a multiple of 32), k-step ks:
//     features 16 ks + 8 g .. +7 = unit 2 ks + g; byte offset
//     256 R0 + (r16 ^ 32 ks)  or  128 R0 + (r8 ^ 32 ks).
//   tr16 / tr8: the transpose read of rows R0 + 16 kk + {4 g + i / 4, +8}
//     (i = l % 16) at columns 32 cb + 16 ((l / 16) % 2) + 4 (i % 4): lane l
//     receives column 32 cb + l % 32 at rows R0 + 16 kk + acc_row(0..7, g),
//     the k-slot order of a 32x32 accumulator; byte offset
//     256 (R0 + 16 kk) + (t16[sec] ^ 64 cb)  (8-unit: 128 (..) + (t8[sec] ^ 64 cb)).
struct LaneOff {
  uint32_t r16, r8, t16[2], t8[2];
};
__device__ __forceinline__ LaneOff lane_offsets(int lane) {
  const int g = lane >> 5, l32 = lane & 31, i16 = lane & 15, mh = (lane >> 4) & 1;
  LaneOff o;
  o.r16 = 256 * l32 + 16 * (g ^ sw16(l32 & 15));
  o.r8 = 128 * l32 + 16 * (g ^ sw8(l32 & 15));
#pragma unroll
  for (int sec = 0; sec < 2; ++sec) {
    const int rr = 4 * g + 8 * sec + (i16 >> 2);   // row within the 16-row k-block
    const int lo = (2 * mh + ((i16 >> 1) & 1)) ^ (g + 2 * sec);
    o.t16[sec] = 256 * rr + 16 * (i16 & 12) + 16 * lo + 8 * (i16 & 1);
    o.t8[sec] = 128 * rr + 64 * ((i16 >> 3) & 1) + 16 * lo + 8 * (i16 & 1);
  }
  return o;
}

__device__ __forceinline__ bf16x8 ld_row16(const char* reg, const LaneOff& o, int R0, int ks) {
  return *reinterpret_cast<const bf16x8*>(reg + (256 * R0 + (o.r16 ^ (32 * ks))));
}
__device__ __forceinline__ bf16x8 ld_row8(const char* reg, const LaneOff& o, int R0, int ks) {
  return *reinterpret_cast<const bf16x8*>(reg + (128 * R0 + (o.r8 ^ (32 * ks))));
}
__device__ __forceinline__ v4s tr4(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)((const lds_char*)p));
}
__device__ __forceinline__ bf16x8 cat8(v4s lo, v4s hi) {
  typedef short v8s __attribute__((ext_vector_type(8)));
  const v8s x = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, x);
}
__device__ __forceinline__ bf16x8 ld_tr16(const char* reg, const LaneOff& o, int R0, int cb) {
  const char* b = reg + 256 * R0;
  return cat8(tr4(b + (o.t16[0] ^ (64 * cb))), tr4(b + (o.t16[1] ^ (64 * cb))));
}
__device__ __forceinline__ bf16x8 ld_tr8(const char* reg, const LaneOff& o, int R0, int cb) {
  const char* b = reg + 128 * R0;
  return cat8(tr4(b + (o.t8[0] ^ (64 * cb))), tr4(b + (o.t8[1] ^ (64 * cb))));
}

// Row of accumulator element i within a 32x32 block, lane half 0 (half g adds 4 g).
__host__ __device__ constexpr int arow0(int i) { return ((i >> 2) << 3) + (i & 3); }

// bf16 pack of accumulator elements 8 kk .. 8 kk + 7 (the k-slots of one
// 16-row k-step when the accumulator is reused as an operand).
__device__ __forceinline__ bf16x8 pack8(const float (&v)[16], int kk) {
  uint4 u;
  u.x = pack_bf16x2(v[8 * kk + 0], v[8 * kk + 1]);
  u.y = pack_bf16x2(v[8 * kk + 2], v[8 * kk + 3]);
  u.z = pack_bf16x2(v[8 * kk + 4], v[8 * kk + 5]);
  u.w = pack_bf16x2(v[8 * kk + 6], v[8 * kk + 7]);
  return as_bf16x8(u);
}

// ---------------------------------------------------------------------------
// Plan: work items {sequence, block of 128 rows} for both passes, longest
// first (counting sort on the item's tile count; ties in any order):
//   dK/dV item (s, b): query tiles 2 b .. ceil(L / 64) - 1
//   dQ item (s, b):    key tiles 0 .. min(2 b + 1, ceil(L / 64) - 1)
// count[0] = number of items (the same for both lists).
// ---------------------------------------------------------------------------
constexpr int kPlanThreads = 1024;
constexpr int kPlanBuckets = 4096;   // tile counts past this share the top bucket
constexpr int kPlanPer = kPlanBuckets / kPlanThreads;

__device__ __forceinline__ int bw_seq_len(const int32_t* cu, int s, int64_t ntok, int64_t* a_out) {
  int64_t a = cu[s], b = cu[s + 1];
  a = a < 0 ? 0 : (a > ntok ? ntok : a);
  b = b < a ? a : (b > ntok ? ntok : b);
  *a_out = a;
  return static_cast<int>(b - a);
}

__global__ void __launch_bounds__(kPlanThreads) bwd_plan_kernel(const int32_t* __restrict__ cu, int nseq,
                                                                int64_t ntok, int2* __restrict__ items_kv,
                                                                int2* __restrict__ items_q,
                                                                int32_t* __restrict__ count) {
  __shared__ int hist[2][kPlanBuckets];
  __shared__ int part[2][kPlanThreads];
  const int tid = threadIdx.x;
  for (int i = tid; i < 2 * kPlanBuckets; i += kPlanThreads) hist[i / kPlanBuckets][i % kPlanBuckets] = 0;
  __syncthreads();
  auto bucket = [](int w) { return w < kPlanBuckets - 1 ? w : kPlanBuckets - 1; };
  for (int s = tid; s < nseq; s += kPlanThreads) {
    int64_t a;
    const int L = bw_seq_len(cu, s, ntok, &a);
    const int nt = (L + kBwTile - 1) / kBwTile, nb = (L + kBwBlock - 1) / kBwBlock;
    for (int b = 0; b < nb; ++b) {
      atomicAdd(&hist[0][bucket(nt - 2 * b)], 1);
      atomicAdd(&hist[1][bucket(min(2 * b + 2, nt))], 1);
    }
  }
  __syncthreads();
  // Thread t owns the kPlanPer buckets ranked kPlanPer t .. from the top;
  // inclusive scan of the per-thread sums, then each bucket's first slot.
  for (int k = 0; k < 2; ++k) {
    int sum = 0;
    for (int j = 0; j < kPlanPer; ++j) sum += hist[k][kPlanBuckets - 1 - (kPlanPer * tid + j)];
    part[k][tid] = sum;
  }
  __syncthreads();
  for (int off = 1; off < kPlanThreads; off <<= 1) {
    const int v0 = tid >= off ? part[0][tid - off] : 0, v1 = tid >= off ? part[1][tid - off] : 0;
    __syncthreads();
    part[0][tid] += v0;
    part[1][tid] += v1;
    __syncthreads();
  }
  for (int k = 0; k < 2; ++k) {
    int run = tid ? part[k][tid - 1] : 0;
    for (int j = 0; j < kPlanPer; ++j) {
      const int idx = kPlanBuckets - 1 - (kPlanPer * tid + j);
      const int c = hist[k][idx];
      hist[k][idx] = run;
      run += c;
    }
  }
  __syncthreads();
  if (tid == 0) count[0] = part[0][kPlanThreads - 1];
  for (int s = tid; s < nseq; s += kPlanThreads) {
    int64_t a;
    const int L = bw_seq_len(cu, s, ntok, &a);
    const int nt = (L + kBwTile - 1) / kBwTile, nb = (L + kBwBlock - 1) / kBwBlock;
    for (int b = 0; b < nb; ++b) {
      items_kv[atomicAdd(&hist[0][bucket(nt - 2 * b)], 1)] = make_int2(s, b);
      items_q[atomicAdd(&hist[1][bucket(min(2 * b + 2, nt))], 1)] = make_int2(s, b);
    }
  }
}

// ---------------------------------------------------------------------------
// Preparation, per (token, head) row of 128: dO~ = dO . sigma(g) (bf16),
// dg = dO . o . (1 - sigma(g)), and {lse log2(e), D = rowsum(dO . o)} into
// lsed [H][T]. 32 threads per row, 8 rows per 256-thread block.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) bwd_prep_kernel(const float* __restrict__ dout, const float* __restrict__ out,
                                                       const uint16_t* __restrict__ gate,
                                                       const float* __restrict__ lse, int heads, int64_t ntok,
                                                       uint16_t* __restrict__ dot, float2* __restrict__ lsed,
                                                       float* __restrict__ dgate) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 8 + (threadIdx.x >> 5);
  const int j = threadIdx.x & 31;
  if (row >= ntok * heads) return;   // whole 32-lane groups leave together
  const int64_t t = row / heads;
  const int h = static_cast<int>(row - t * heads);
  const int64_t col = row * kV + 4 * j;
  const float4 dv = *reinterpret_cast<const float4*>(dout + col);
  const float4 ov = *reinterpret_cast<const float4*>(out + col);
  float sg0 = 1.0f, sg1 = 1.0f, sg2 = 1.0f, sg3 = 1.0f;
  if (gate) {
    const uint2 gb = *reinterpret_cast<const uint2*>(gate + col);
    sg0 = sigmoidf_(bf16lo(gb.x));
    sg1 = sigmoidf_(bf16hi(gb.x));
    sg2 = sigmoidf_(bf16lo(gb.y));
    sg3 = sigmoidf_(bf16hi(gb.y));
    *reinterpret_cast<float4*>(dgate + col) = make_float4(dv.x * ov.x * (1.0f - sg0), dv.y * ov.y * (1.0f - sg1),
                                                          dv.z * ov.z * (1.0f - sg2), dv.w * ov.w * (1.0f - sg3));
  }
  *reinterpret_cast<uint2*>(dot + col) =
      make_uint2(pack_bf16x2(dv.x * sg0, dv.y * sg1), pack_bf16x2(dv.z * sg2, dv.w * sg3));
  float pr = dv.x * ov.x + dv.y * ov.y + dv.z * ov.z + dv.w * ov.w;
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) pr += __shfl_xor(pr, o, 64);
  if (j == 0) lsed[static_cast<int64_t>(h) * ntok + t] = make_float2(lse[static_cast<int64_t>(h) * ntok + t] * kLog2e, pr);
}

// ---------------------------------------------------------------------------
// dK/dV pass. Block x = item * heads + head.
// ---------------------------------------------------------------------------
__shared__ __align__(1024) char g_bw_lds[2 * kKvStage];

// A tile body is one fixed sequence of matrix-core products ("ops") in four
// phases, each a scheduling region of its own:
//   1  score products of block 0: X0 (wide, 12 k-steps) and Y0 (narrow, 8)
//      alternating, X0's last four alone
//   2  the same for block 1, while the VALU turns block 0's scores into
//      bf16 operands (softmax)
//   3  gradient products of block 0, while the VALU does block 1's softmax
//   4  gradient products of block 1
// Each op's LDS operand read is issued kAhead ops earlier in program order
// (across phase boundaries), and the phases' instruction groups interleave
// one product with its reads and a share of the VALU work.
struct TileOp {
  int kind, blk, ks, cb;   // kind 0: wide score, 1: narrow score, 2 / 3: gradient products
};
__host__ __device__ constexpr TileOp score_op(int blk, int r) {
  return r < 16 ? TileOp{r & 1, blk, r >> 1, 0} : TileOp{0, blk, 8 + (r - 16), 0};
}
constexpr int kScoreOps = 20;   // per block
constexpr int kAhead = 4;

// Instruction groups of one phase: an initial batch of reads, then per
// product one MFMA, its share of reads and of VALU work.
template <int NOPS, int FIRST_DS, int DS_PER, int VALU_PER>
__device__ __forceinline__ void phase_schedule() {
  if constexpr (FIRST_DS > 0) __builtin_amdgcn_sched_group_barrier(0x100, FIRST_DS, 0);
  static_for<0, NOPS>([&](auto) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (DS_PER > 0) __builtin_amdgcn_sched_group_barrier(0x100, DS_PER, 0);
    if constexpr (VALU_PER > 0) __builtin_amdgcn_sched_group_barrier(0x002, VALU_PER, 0);
  });
  __builtin_amdgcn_sched_barrier(0);
}

// dK/dV tile ops: phases 1, 2 score products of blocks 0, 1; phases 3, 4
// gradient products of blocks 0, 1 (k-step kk of the block, then per kk the
// four dV column blocks and the six dK column blocks).
__host__ __device__ constexpr TileOp kv_op(int e) {
  if (e < 2 * kScoreOps) return score_op(e / kScoreOps, e % kScoreOps);
  const int blk = (e - 2 * kScoreOps) / 20, r = (e - 2 * kScoreOps) % 20, kk = r / 10, j = r % 10;
  return j < 4 ? TileOp{2, blk, kk, j} : TileOp{3, blk, kk, j - 4};
}
constexpr int kKvOps = 80;

// One query tile for the wave's 32 keys. MASK: P is kept where
// (unsigned)(kd + row) < span for the element's row in the tile; with
// kd = q0 + 4 g - key and span = max(L - key, 0) that is key <= query < L.
// Without MASK every element is kept (the tile lies past the block's keys
// and before L). The leading asm names the variant in the assembly listing.
template <bool MASK>
__device__ __forceinline__ void dkv_tile(const char* st, int lane, const bf16x8 (&kf)[12], const bf16x8 (&vf)[8],
                                         f32x16 (&dk)[6], f32x16 (&dv)[4], float c, int kd, int span) {
  asm volatile("; dK/dV tile, masked: %0" ::"n"(MASK ? 1 : 0));
  // the lane's LDS offsets, formed here from an opaque copy of the lane index:
  // held across the tile loop they were spilled and reloaded behind waits
  int lane_o = lane;
  asm volatile("" : "+v"(lane_o));
  const LaneOff o = lane_offsets(lane_o);
  const char* qc = st;
  const char* qr = st + kReg16;
  const char* od = st + kReg16 + kReg8;
  const char* info = st + 2 * kReg16 + kReg8;
  const int g = lane >> 5;
  f32x16 s[2], dp[2];
  bf16x8 pa[2][2], da[2][2];
  float4 inf[2][8];
  auto rd = [&](auto E) -> bf16x8 {
    constexpr TileOp op = kv_op(E);
    if constexpr (op.kind == 0) {
      if constexpr (op.ks < 8) return ld_row16(qc, o, 32 * op.blk, op.ks);
      else return ld_row8(qr, o, 32 * op.blk, op.ks - 8);
    } else if constexpr (op.kind == 1) {
      return ld_row16(od, o, 32 * op.blk, op.ks);
    } else if constexpr (op.kind == 2) {
      return ld_tr16(od, o, 32 * op.blk + 16 * op.ks, op.cb);
    } else {
      if constexpr (op.cb < 4) return ld_tr16(qc, o, 32 * op.blk + 16 * op.ks, op.cb);
      else return ld_tr8(qr, o, 32 * op.blk + 16 * op.ks, op.cb - 4);
    }
  };
  // {lse log2(e), D} of the 16 rows of block b the lane holds: rows 8 j + 4 g .. +3
  auto rd_info = [&](auto B) {
    static_for<0, 4>([&](auto J) {
      const float4* ip = reinterpret_cast<const float4*>(info + 8 * (32 * B + 8 * J + 4 * g));
      inf[B][2 * J] = ip[0];
      inf[B][2 * J + 1] = ip[1];
    });
  };
  // P and dS' = P (dP - D) of block b as bf16 operands (k-step kk: elements 8 kk .. 8 kk + 7)
  auto softmax = [&](auto B) {
    float p[16], d[16];
    static_for<0, 16>([&](auto II) {
      constexpr int i = II, J = i / 4, E = i % 4;
      const float4 v = inf[B][2 * J + E / 2];
      const float l2 = (E & 1) ? v.z : v.x, dd = (E & 1) ? v.w : v.y;
      constexpr int ci = 32 * B + arow0(i);
      float pv = fast_exp2(fmaf(s[B][i], c, -l2));
      if constexpr (MASK) pv = static_cast<unsigned>(kd + ci) < static_cast<unsigned>(span) ? pv : 0.0f;
      p[i] = pv;
      d[i] = pv * (dp[B][i] - dd);
    });
    pa[B][0] = pack8(p, 0);
    pa[B][1] = pack8(p, 1);
    da[B][0] = pack8(d, 0);
    da[B][1] = pack8(d, 1);
  };
  static_for<0, 2>([&](auto B) {
    s[B] = f32x16{};
    dp[B] = f32x16{};
  });
  bf16x8 buf[kAhead];
  static_for<0, kAhead>([&](auto E) { buf[E] = rd(E); });
  static_for<0, kKvOps>([&](auto E) {
    constexpr TileOp op = kv_op(E);
    if constexpr (E == kScoreOps) phase_schedule<kScoreOps, kAhead, 1, 0>();
    if constexpr (E == 2 * kScoreOps) phase_schedule<kScoreOps, 8, 1, 7>();
    if constexpr (E == 3 * kScoreOps) phase_schedule<20, 8, 2, 7>();
    if constexpr (E == kScoreOps) rd_info(std::integral_constant<int, 0>{});
    if constexpr (E == 2 * kScoreOps) rd_info(std::integral_constant<int, 1>{});
    const bf16x8 x = buf[E % kAhead];
    if constexpr (E + kAhead < kKvOps) buf[E % kAhead] = rd(std::integral_constant<int, E + kAhead>{});
    if constexpr (op.kind == 0) s[op.blk] = mfma32(x, kf[op.ks], s[op.blk]);
    else if constexpr (op.kind == 1) dp[op.blk] = mfma32(x, vf[op.ks], dp[op.blk]);
    else if constexpr (op.kind == 2) dv[op.cb] = mfma32(pa[op.blk][op.ks], x, dv[op.cb]);
    else dk[op.cb] = mfma32(da[op.blk][op.ks], x, dk[op.cb]);
    if constexpr (E == 2 * kScoreOps - 1) softmax(std::integral_constant<int, 0>{});
    if constexpr (E == 3 * kScoreOps - 1) softmax(std::integral_constant<int, 1>{});
  });
  phase_schedule<20, 0, 2, 0>();
}

__global__ void __launch_bounds__(kBwThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) bwd_dkv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const uint16_t* __restrict__ ksh,
    const uint16_t* __restrict__ dot, const float2* __restrict__ lsed, const int32_t* __restrict__ cu,
    const int2* __restrict__ items, const int32_t* __restrict__ count, int heads, int64_t ntok, float scale,
    uint16_t* __restrict__ dkv, float* __restrict__ dksp) {
  const int h = static_cast<int>(blockIdx.x % heads);
  const int item = static_cast<int>(blockIdx.x / heads);
  if (item >= count[0]) return;
  const int2 it = items[item];
  int64_t a;
  const int L = bw_seq_len(cu, it.x, ntok, &a);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int kb0 = kBwBlock * it.y, kw0 = kb0 + 32 * w;
  const int key = kw0 + l32;   // this lane's key (sequence-relative)
  const int span = max(L - key, 0);
  const int64_t HQ = static_cast<int64_t>(heads) * kD * 2, HO = static_cast<int64_t>(heads) * kV * 2;

  const int nq = (L + kBwTile - 1) / kBwTile;
  const int qt_lo = kb0 / kBwTile;
  const int ntiles = nq - qt_lo;
  const uint32_t lds0 = lds_off(g_bw_lds);
  auto issue = [&](int j, int stage) {   // copies of query tile nq - 1 - j into a stage
    const int64_t t0 = a + static_cast<int64_t>(kBwTile) * (nq - 1 - j);
    const uint32_t base = lds0 + stage * kKvStage;
    const int64_t rows_left = ntok - t0;
    const u32x4 rq = bw_rsrc(q + (t0 * heads + h) * kD, rows_left * HQ - h * (kD * 2));
    copy16(rq, HQ, 0, base, w, lane);
    copy8(rq, HQ, kN * 2, base + kReg16, w, lane);
    const u32x4 ro = bw_rsrc(dot + (t0 * heads + h) * kV, rows_left * HO - h * (kV * 2));
    copy16(ro, HO, 0, base + kReg16 + kReg8, w, lane);
    if (w == 0) {
      const u32x4 ri = bw_rsrc(lsed + static_cast<int64_t>(h) * ntok + t0, rows_left * 8);
      bw_dma16(ri, 16 * lane, base + 2 * kReg16 + kReg8);
    }
  };
  if (ntiles > 0) issue(0, 0);

  // the wave's K (K^C then k^S) and V fragments: key row, features 16 ks + 8 g ..
  bf16x8 kf[12], vf[8];
  {
    const bool ok = key < L;
    const int64_t t = a + key;
    const uint16_t* kr = kv + (t * heads + h) * (kN + kV) + 8 * g;
    const uint16_t* sr = ksh + t * kS + 8 * g;
    static_for<0, 8>([&](auto KS) {
      kf[KS] = ok ? as_bf16x8(ldg16(kr + 16 * KS)) : bf16x8{};
      vf[KS] = ok ? as_bf16x8(ldg16(kr + kN + 16 * KS)) : bf16x8{};
    });
    static_for<0, 4>([&](auto KS) { kf[8 + KS] = ok ? as_bf16x8(ldg16(sr + 16 * KS)) : bf16x8{}; });
  }
  f32x16 dk[6], dv[4];
  static_for<0, 6>([&](auto I) { dk[I] = f32x16{}; });
  static_for<0, 4>([&](auto I) { dv[I] = f32x16{}; });
  const float c = scale * kLog2e;
  wait_vmcnt<0>();
  bw_barrier();
  // query tile j: the next tile's copies, the tile, its landing and the barrier
  auto run_tile = [&](int j, auto M) {
    constexpr bool kMask = decltype(M)::value;
    const int stage = j & 1;
    if (j + 1 < ntiles) issue(j + 1, stage ^ 1);
    const int q0 = kBwTile * (nq - 1 - j);
    const char* st = g_bw_lds + stage * kKvStage;
    if constexpr (kMask) {
      if (q0 + kBwTile - 1 >= kw0)   // else every query of the tile precedes the wave's keys
        dkv_tile<true>(st, lane, kf, vf, dk, dv, c, q0 + 4 * g - key, span);
    } else {
      dkv_tile<false>(st, lane, kf, vf, dk, dv, c, 0, 0);
    }
    wait_vmcnt<0>();
    bw_barrier();
  };
  // Tiles 0 .. ntiles - 3 start at or past the block's first key + 128, so
  // no wave masks them for causality; tile 0 alone can reach past L (when L is
  // not a multiple of 64) and then takes the masked body. The last two tiles
  // are the diagonal. The loops are separate so that the main one holds only
  // the unmasked body (the mask select is 16 VALU ops per accumulator block).
  int jt = 0;
  if (ntiles > 0 && kBwTile * nq > L) run_tile(jt++, std::true_type{});
  for (; jt < ntiles - 2; ++jt) run_tile(jt, std::false_type{});
  for (; jt < ntiles; ++jt) run_tile(jt, std::true_type{});
  // dV rows (bf16), dK^C rows scaled (bf16), k^S part scaled into the per-head partials (fp32):
  // accumulator block b: lane = column 32 b + l32, element i = key kw0 + acc_row(i, g)
  static_for<0, 16>([&](auto II) {
    constexpr int I = II;
    const int kr = kw0 + acc_row(I, g);
    if (kr < L) {
      const int64_t t = a + kr;
      uint16_t* dr = dkv + (t * heads + h) * (kN + kV) + l32;
      static_for<0, 4>([&](auto B) {
        dr[32 * B] = f32_to_bf16(scale * dk[B][I]);
        dr[kN + 32 * B] = f32_to_bf16(dv[B][I]);
      });
      float* sp = dksp + (static_cast<int64_t>(h) * ntok + t) * kS + l32;
      sp[0] = scale * dk[4][I];
      sp[32] = scale * dk[5][I];
    }
  });
}

// ---------------------------------------------------------------------------
// dQ pass. Block x = item * heads + head.
// ---------------------------------------------------------------------------
// dQ tile ops: phases 1, 2 score products of key blocks 0, 1; phases 3, 4
// dQ products of key blocks 0, 1 (k-step kk, then the six column blocks).
__host__ __device__ constexpr TileOp q_op(int e) {
  if (e < 2 * kScoreOps) return score_op(e / kScoreOps, e % kScoreOps);
  const int blk = (e - 2 * kScoreOps) / 12, r = (e - 2 * kScoreOps) % 12;
  return TileOp{3, blk, r / 6, r % 6};
}
constexpr int kQOps = 64;

// One key tile for the wave's 32 queries (this lane's lse log2(e) l2 and
// D dd). MASK: P is kept where the element's row (key) in the tile is <= m;
// with m = query - k0 - 4 g that is key <= query. Without MASK every element
// is kept (the tile ends before the block's first query).
template <bool MASK>
__device__ __forceinline__ void dq_tile(const char* st, const LaneOff& o, const bf16x8 (&qf)[12],
                                        const bf16x8 (&of)[8], f32x16 (&dq)[6], float c, float l2, float dd, int m) {
  asm volatile("; dQ tile, masked: %0" ::"n"(MASK ? 1 : 0));
  const char* kc = st;
  const char* kr = st + kReg16;
  const char* vt = st + kReg16 + kReg8;
  f32x16 s[2], dp[2];
  bf16x8 da[2][2];
  auto rd = [&](auto E) -> bf16x8 {
    constexpr TileOp op = q_op(E);
    if constexpr (op.kind == 0) {
      if constexpr (op.ks < 8) return ld_row16(kc, o, 32 * op.blk, op.ks);
      else return ld_row8(kr, o, 32 * op.blk, op.ks - 8);
    } else if constexpr (op.kind == 1) {
      return ld_row16(vt, o, 32 * op.blk, op.ks);
    } else {
      if constexpr (op.cb < 4) return ld_tr16(kc, o, 32 * op.blk + 16 * op.ks, op.cb);
      else return ld_tr8(kr, o, 32 * op.blk + 16 * op.ks, op.cb - 4);
    }
  };
  auto softmax = [&](auto B) {
    float d[16];
    static_for<0, 16>([&](auto II) {
      constexpr int i = II;
      constexpr int ci = 32 * B + arow0(i);
      float pv = fast_exp2(fmaf(s[B][i], c, -l2));
      if constexpr (MASK) pv = ci <= m ? pv : 0.0f;
      d[i] = pv * (dp[B][i] - dd);
    });
    da[B][0] = pack8(d, 0);
    da[B][1] = pack8(d, 1);
  };
  static_for<0, 2>([&](auto B) {
    s[B] = f32x16{};
    dp[B] = f32x16{};
  });
  bf16x8 buf[kAhead];
  static_for<0, kAhead>([&](auto E) { buf[E] = rd(E); });
  static_for<0, kQOps>([&](auto E) {
    constexpr TileOp op = q_op(E);
    if constexpr (E == kScoreOps) phase_schedule<kScoreOps, kAhead, 1, 0>();
    if constexpr (E == 2 * kScoreOps) phase_schedule<kScoreOps, 0, 1, 5>();
    if constexpr (E == 2 * kScoreOps + 12) phase_schedule<12, 0, 2, 7>();
    const bf16x8 x = buf[E % kAhead];
    if constexpr (E + kAhead < kQOps) buf[E % kAhead] = rd(std::integral_constant<int, E + kAhead>{});
    if constexpr (op.kind == 0) s[op.blk] = mfma32(x, qf[op.ks], s[op.blk]);
    else if constexpr (op.kind == 1) dp[op.blk] = mfma32(x, of[op.ks], dp[op.blk]);
    else dq[op.cb] = mfma32(da[op.blk][op.ks], x, dq[op.cb]);
    if constexpr (E == 2 * kScoreOps - 1) softmax(std::integral_constant<int, 0>{});
    if constexpr (E == 2 * kScoreOps + 11) softmax(std::integral_constant<int, 1>{});
  });
  phase_schedule<12, 0, 2, 0>();
}

__global__ void __launch_bounds__(kBwThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const uint16_t* __restrict__ ksh,
    const uint16_t* __restrict__ dot, const float2* __restrict__ lsed, const int32_t* __restrict__ cu,
    const int2* __restrict__ items, const int32_t* __restrict__ count, int heads, int64_t ntok, float scale,
    float* __restrict__ dq) {
  const int h = static_cast<int>(blockIdx.x % heads);
  const int item = static_cast<int>(blockIdx.x / heads);
  if (item >= count[0]) return;
  const int2 it = items[item];
  int64_t a;
  const int L = bw_seq_len(cu, it.x, ntok, &a);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int qb0 = kBwBlock * it.y, qw0 = qb0 + 32 * w;
  const int qrow = qw0 + l32;   // this lane's query (sequence-relative)
  const LaneOff o = lane_offsets(lane);
  const int64_t HK = static_cast<int64_t>(heads) * (kN + kV) * 2;

  const int nq = (L + kBwTile - 1) / kBwTile;
  const int ntiles = min(nq, (qb0 + kBwBlock - 1) / kBwTile + 1);
  const uint32_t lds0 = lds_off(g_bw_lds);
  auto issue = [&](int j, int stage) {   // copies of key tile j into a stage
    const int64_t t0 = a + static_cast<int64_t>(kBwTile) * j;
    const uint32_t base = lds0 + stage * kQStage;
    const int64_t rows_left = ntok - t0;
    const u32x4 rk = bw_rsrc(kv + (t0 * heads + h) * (kN + kV), rows_left * HK - h * ((kN + kV) * 2));
    copy16(rk, HK, 0, base, w, lane);
    copy16(rk, HK, kN * 2, base + kReg16 + kReg8, w, lane);
    const u32x4 rs = bw_rsrc(ksh + t0 * kS, rows_left * (kS * 2));
    copy8(rs, kS * 2, 0, base + kReg16, w, lane);
  };
  if (ntiles > 0) issue(0, 0);

  bf16x8 qf[12], of[8];
  float l2 = 0.0f, dd = 0.0f;
  {
    const bool ok = qrow < L;
    const int64_t t = a + qrow;
    const uint16_t* qp = q + (t * heads + h) * kD + 8 * g;
    const uint16_t* op = dot + (t * heads + h) * kV + 8 * g;
    static_for<0, 12>([&](auto KS) { qf[KS] = ok ? as_bf16x8(ldg16(qp + 16 * KS)) : bf16x8{}; });
    static_for<0, 8>([&](auto KS) { of[KS] = ok ? as_bf16x8(ldg16(op + 16 * KS)) : bf16x8{}; });
    if (ok) {
      const float2 x = lsed[static_cast<int64_t>(h) * ntok + t];
      l2 = x.x;
      dd = x.y;
    }
  }
  f32x16 acc[6];
  static_for<0, 6>([&](auto I) { acc[I] = f32x16{}; });
  const float c = scale * kLog2e;
  wait_vmcnt<0>();
  bw_barrier();
  // key tile j: the next tile's copies, the tile, its landing and the barrier
  auto run_tile = [&](int j, auto M) {
    constexpr bool kMask = decltype(M)::value;
    const int stage = j & 1;
    if (j + 1 < ntiles) issue(j + 1, stage ^ 1);
    const int k0 = kBwTile * j;
    const char* st = g_bw_lds + stage * kQStage;
    if constexpr (kMask) {
      if (k0 <= qw0 + 31)   // else every key of the tile follows the wave's queries
        dq_tile<true>(st, o, qf, of, acc, c, l2, dd, qrow - k0 - 4 * g);
    } else {
      dq_tile<false>(st, o, qf, of, acc, c, l2, dd, 0);
    }
    wait_vmcnt<0>();
    bw_barrier();
  };
  // key tiles before the block's first query need no mask for any wave; the
  // last (at most) two are the diagonal
  const int j_unmasked = min(ntiles, qb0 / kBwTile);
  int jt = 0;
  for (; jt < j_unmasked; ++jt) run_tile(jt, std::false_type{});
  for (; jt < ntiles; ++jt) run_tile(jt, std::true_type{});
  // accumulator block b: lane = feature 32 b + l32, element i = query qw0 + acc_row(i, g)
  static_for<0, 16>([&](auto II) {
    constexpr int I = II;
    const int qr = qw0 + acc_row(I, g);
    if (qr < L) {
      float* dr = dq + ((a + qr) * heads + h) * kD + l32;
      static_for<0, 6>([&](auto B) { dr[32 * B] = scale * acc[B][I]; });
    }
  });
}

// dk^S[t][j] = sum over heads of the per-head partials.
__global__ void __launch_bounds__(256) bwd_dks_kernel(const float* __restrict__ dksp, int heads, int64_t ntok,
                                                      float* __restrict__ dks) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= ntok * kS) return;
  float s = 0.0f;
  for (int h = 0; h < heads; ++h) s += dksp[static_cast<int64_t>(h) * ntok * kS + i];
  dks[i] = s;
}

// out[i] = sum over the split-K partials part[c][i], c < nsplit (n a multiple of 4).
__global__ void __launch_bounds__(256) bwd_sum_kernel(const float* __restrict__ part, int nsplit, int64_t n,
                                                      float* __restrict__ out) {
  const int64_t i = 4 * (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x);
  if (i >= n) return;
  float4 s = *reinterpret_cast<const float4*>(part + i);
  for (int c = 1; c < nsplit; ++c) {
    const float4 v = *reinterpret_cast<const float4*>(part + c * n + i);
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  }
  *reinterpret_cast<float4*>(out + i) = s;
}

// Split of a long-K GEMM with few 256 x 256 output tiles: enough K chunks
// (each a multiple of 128) to give about 512 workgroups, at most 16.
inline int gemm_split(int64_t tiles, int64_t kblocks) {
  int sp = static_cast<int>(std::min<int64_t>(16, std::max<int64_t>(1, 512 / std::max<int64_t>(tiles, 1))));
  while (sp > 1 && kblocks % sp) --sp;
  return sp;
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

inline int64_t round128(int64_t x) { return (x + 127) / 128 * 128; }

}  // namespace

BackwardWs backward_ws_layout(int heads, int64_t ntok, int nseq) {
  BackwardWs w{};
  const size_t T = static_cast<size_t>(ntok), Tp = static_cast<size_t>(round128(ntok));
  const size_t H = static_cast<size_t>(heads), HW = H * (kN + kV);
  w.items = (ntok + kBwBlock - 1) / kBwBlock + nseq;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes, 256); return o; };
  w.kv = take(T * HW * 2);
  w.dot = take(T * H * kV * 2);
  w.lsed = take(H * T * 8);
  w.dkv = take(T * HW * 2);
  w.dkvT = take(HW * Tp * 2);
  w.wT = take(HW * kR * 2);
  w.ckvT = take(static_cast<size_t>(kR) * Tp * 2);
  w.dksp = take(H * T * kS * 4);
  // split-K partials of the two weight products (one at a time)
  const int64_t tiles_c = (ntok + 255) / 256 * 2, tiles_w = (static_cast<int64_t>(HW) + 255) / 256 * 2;
  w.split_c = gemm_split(tiles_c, static_cast<int64_t>(HW) / 128);
  w.split_w = gemm_split(tiles_w, static_cast<int64_t>(Tp) / 128);
  w.part = take(std::max(w.split_c > 1 ? w.split_c * T * kR * 4 : 0, w.split_w > 1 ? w.split_w * HW * kR * 4 : 0));
  w.items_kv = take(static_cast<size_t>(w.items) * 8);
  w.items_q = take(static_cast<size_t>(w.items) * 8);
  w.count = take(16);
  w.total = off;
  return w;
}

hipError_t launch_prefill_backward_bf16(int heads, float scale, const void* q, const void* ckv, const void* ks,
                                        const void* w_kv_b, const void* gate, const int32_t* cu, int nseq,
                                        int64_t ntok, const float* out, const float* lse, const float* dout,
                                        float* dq, float* dckv, float* dks, float* dw, float* dgate, void* ws,
                                        hipStream_t st) {
  const BackwardWs W = backward_ws_layout(heads, ntok, nseq);
  char* base = static_cast<char*>(ws);
  auto b16 = [&](size_t o) { return reinterpret_cast<uint16_t*>(base + o); };
  auto f32 = [&](size_t o) { return reinterpret_cast<float*>(base + o); };
  const int HW = heads * (kN + kV);
  const int64_t Tp = round128(ntok);
  const int T = static_cast<int>(ntok);
  int2* items_kv = reinterpret_cast<int2*>(base + W.items_kv);
  int2* items_q = reinterpret_cast<int2*>(base + W.items_q);
  int32_t* count = reinterpret_cast<int32_t*>(base + W.count);
  float2* lsed = reinterpret_cast<float2*>(base + W.lsed);
  hipError_t e;
#define BW_CHECK()                    \
  do {                                \
    e = hipGetLastError();            \
    if (e != hipSuccess) return e;    \
  } while (0)
  {
    TimedScope ts_("bw_plan", st);
    hipLaunchKernelGGL(bwd_plan_kernel, dim3(1), dim3(kPlanThreads), 0, st, cu, nseq, ntok, items_kv, items_q, count);
  }
  BW_CHECK();
  // [K^C | V] of every head: c^KV W_UKV^T-rows
  {
    const GemmSpec p{static_cast<const uint16_t*>(w_kv_b), b16(W.kv), kR, HW, 0, 0, HW};
    e = launch_gemm_bf16(false, static_cast<const uint16_t*>(ckv), kR, 0, T, kR, 1, 1, &p, "bw_expand", st);
    if (e != hipSuccess) return e;
  }
  {
    TimedScope ts_("bw_prep", st);
    const int64_t rows = ntok * heads;
    hipLaunchKernelGGL(bwd_prep_kernel, dim3(static_cast<unsigned>((rows + 7) / 8)), dim3(256), 0, st, dout, out,
                       static_cast<const uint16_t*>(gate), lse, heads, ntok, b16(W.dot), lsed, dgate);
  }
  BW_CHECK();
  const unsigned blocks = static_cast<unsigned>(W.items * heads);
  {
    TimedScope ts_("bw_dkv", st);
    hipLaunchKernelGGL(bwd_dkv_kernel, dim3(blocks), dim3(kBwThreads), 0, st, static_cast<const uint16_t*>(q),
                       b16(W.kv), static_cast<const uint16_t*>(ks), b16(W.dot), lsed, cu, items_kv, count, heads,
                       ntok, scale, b16(W.dkv), f32(W.dksp));
  }
  BW_CHECK();
  {
    TimedScope ts_("bw_dq", st);
    hipLaunchKernelGGL(bwd_dq_kernel, dim3(blocks), dim3(kBwThreads), 0, st, static_cast<const uint16_t*>(q),
                       b16(W.kv), static_cast<const uint16_t*>(ks), b16(W.dot), lsed, cu, items_q, count, heads, ntok,
                       scale, dq);
  }
  BW_CHECK();
  {
    TimedScope ts_("bw_dks", st);
    hipLaunchKernelGGL(bwd_dks_kernel, dim3(static_cast<unsigned>((ntok * kS + 255) / 256)), dim3(256), 0, st,
                       f32(W.dksp), heads, ntok, dks);
  }
  BW_CHECK();
  {
    TimedScope ts_("bw_transpose", st);
    hipLaunchKernelGGL(bw_transpose_kernel, dim3((HW + 63) / 64, kR / 64, 1), dim3(256), 0, st,
                       static_cast<const uint16_t*>(w_kv_b), static_cast<int64_t>(HW), static_cast<int64_t>(HW), kR,
                       int64_t{0}, int64_t{0}, b16(W.wT));
    hipLaunchKernelGGL(bw_transpose_kernel, dim3(static_cast<unsigned>(Tp / 64), kR / 64, 1), dim3(256), 0, st,
                       static_cast<const uint16_t*>(ckv), ntok, Tp, kR, int64_t{0}, int64_t{0}, b16(W.ckvT));
    hipLaunchKernelGGL(bw_transpose_kernel, dim3(static_cast<unsigned>(Tp / 64), (HW + 63) / 64, 1), dim3(256), 0,
                       st, b16(W.dkv), ntok, Tp, HW, int64_t{0}, int64_t{0}, b16(W.dkvT));
  }
  BW_CHECK();
  {  // dc^KV = dKV W_UKV (through W^T rows) and dW = dKV^T c^KV (fp32), split over K into
     // partials summed afterwards when the outputs have few tiles
    const int sc = W.split_c, sw = W.split_w;
    const int64_t kc = HW / sc, kw = Tp / sw;
    const GemmSpec pc{b16(W.wT), sc > 1 ? f32(W.part) : dckv, HW, kR, kc, ntok * kR, kR};
    e = launch_gemm_bf16(true, b16(W.dkv), HW, kc, T, static_cast<int>(kc), sc, 1, &pc, "bw_weights", st);
    if (e != hipSuccess) return e;
    if (sc > 1) {
      TimedScope ts_("bw_weights", st);
      const int64_t n = ntok * kR;
      hipLaunchKernelGGL(bwd_sum_kernel, dim3(static_cast<unsigned>((n / 4 + 255) / 256)), dim3(256), 0, st,
                         f32(W.part), sc, n, dckv);
      BW_CHECK();
    }
    const GemmSpec pw{b16(W.ckvT), sw > 1 ? f32(W.part) : dw, Tp, kR, kw, static_cast<int64_t>(HW) * kR, kR};
    e = launch_gemm_bf16(true, b16(W.dkvT), Tp, kw, HW, static_cast<int>(kw), sw, 1, &pw, "bw_weights", st);
    if (e != hipSuccess) return e;
    if (sw > 1) {
      TimedScope ts_("bw_weights", st);
      const int64_t n = static_cast<int64_t>(HW) * kR;
      hipLaunchKernelGGL(bwd_sum_kernel, dim3(static_cast<unsigned>((n / 4 + 255) / 256)), dim3(256), 0, st,
                         f32(W.part), sw, n, dw);
      BW_CHECK();
    }
  }
#undef BW_CHECK
  return hipSuccess;
}

}  // namespace mla
