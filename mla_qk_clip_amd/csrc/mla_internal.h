// Host-side launch helpers shared between the C ABI front end and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

// Kimi K3 head shape compiled into the bf16 MFMA kernels.
constexpr int kR = 512;   // kv_rank
constexpr int kS = 64;    // shared key width
constexpr int kN = 128;   // nope width
constexpr int kV = 128;   // value width
constexpr int kD = kN + kS;

// Prefill (bf16) tiling.
constexpr int kPrefBM = 128;  // queries per attention workgroup (two workgroups per CU)
constexpr int kPrefBN = 64;   // keys per inner tile
constexpr int kSeqPad = 64;   // per-sequence padding of the expanded K^C / V^T

// Absorbed (bf16) split-K.
constexpr int kDecSplits = 256;  // workgroups of the split kernel
constexpr int kDecRows = 32;     // cache rows per inner tile
constexpr int kDecHeadsPerWg = 96;  // 3 compute waves x 32 heads
constexpr int kDecMaxHeads = 128;

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace layout of the bf16 prefill. Sequences are padded to multiples of
// 64 rows; padded row p belongs to 64-row key tile p / 64 and the expanded
// operands are stored tile-blocked in the order the attention kernel copies
// them into LDS (1 KB = 64 x 16 bytes per block, padding rows zero):
//   kc [H][tile][16 units][64 rows][8]   K^C, unit u = features kperm(8u..8u+7),
//                                        kperm(n) = (n & ~15) | vperm16(n & 15)
//   vt [H][tile][8 units][128 d][8]      V^T, unit u = keys at permuted
//                                        positions 8u..8u+7 of the tile
//   ksp[tile][8 units][64 rows][8]       k^S (shared by all heads)
struct PrefillWs {
  size_t kc, vt, ksp, pcu, order, toff, hdr, rowmax, aux, cand, qx, qmeta, total;
  int64_t npad_max;
};
constexpr int kTileElems = kPrefBN * kN;  // elements of one K^C (or V^T) tile of one head
// aux[h][0] = approximate (raw, unscaled) head max logit, aux[h][1] = max |q_t|^2,
// aux[h][2] = max |K^C_s|^2 (bf16 values), aux[h][3] unused; aux[H][0] = max |k^S_s|^2.
constexpr int kAuxStride = 4;
// Max-logit refinement state (int32): [0] listed rows of all heads (they are
// numbered densely), [1..3] unused, then per head the number of its rows that
// reached the threshold (kCandHeadCount + h); a head with more than kRefRows
// falls back to the approximate maximum.
constexpr int kRefRows = 64;
constexpr int kCandHeadCount = 4;
inline PrefillWs prefill_ws_layout(int heads, int64_t ntok, int nseq) {
  PrefillWs w{};
  w.npad_max = static_cast<int64_t>(align_up(static_cast<size_t>(ntok + static_cast<int64_t>(kSeqPad) * nseq), 256));
  size_t off = 0;
  w.kc = off; off = align_up(off + static_cast<size_t>(heads) * w.npad_max * kN * 2, 256);
  w.vt = off; off = align_up(off + static_cast<size_t>(heads) * w.npad_max * kV * 2, 256);
  w.ksp = off; off = align_up(off + static_cast<size_t>(w.npad_max) * kS * 2, 256);
  w.pcu = off; off = align_up(off + static_cast<size_t>(nseq + 1) * 4, 256);
  w.order = off; off = align_up(off + static_cast<size_t>(nseq + 1) * 4, 256);
  w.toff = off; off = align_up(off + static_cast<size_t>(nseq + 1) * 4, 256);
  w.hdr = off; off = align_up(off + 64, 256);
  w.rowmax = off; off = align_up(off + static_cast<size_t>(heads) * ntok * 4, 256);
  w.aux = off; off = align_up(off + static_cast<size_t>(heads + 1) * kAuxStride * 4, 256);
  w.cand = off; off = align_up(off + static_cast<size_t>(kCandHeadCount + heads) * 4, 256);
  // listed rows of all heads, numbered densely: q_abs as bf16 hi | lo parts, and {row, sequence start, head}
  w.qx = off; off = align_up(off + static_cast<size_t>(heads) * kRefRows * (kR + kS) * 2 * 2, 256);
  w.qmeta = off; off = align_up(off + static_cast<size_t>(heads) * kRefRows * 16, 256);
  w.total = off;
  return w;
}

// Workspace layout of the fp32 prefill: K^C [H][Ntok][N], V [H][Ntok][V].
inline size_t prefill_f32_ws(int heads, int64_t ntok, int N, int V) {
  return align_up(static_cast<size_t>(heads) * ntok * (N + V) * 4, 256);
}

// Workspace layout of the bf16 absorbed path.
// Workspace of the bf16 absorbed form. Besides q_abs, the prefix sums and
// the split-K partials it holds what the max-logit refinement needs:
//   qlo  [bt][H][R]  bf16 rounding residual of the first R entries of q_abs
//   dlb  [G][H]      per split workgroup and head: a lower bound of the
//                    head's exact max logit (raw) from the workgroup's tiles
//   dcnt [G][H]      live entries in dent (kDecList + 1: the list overflowed)
//   dent [G][H][kDecList]  {virtual sequence, first row in the sequence,
//                    rows, bits of an upper bound of the tile's exact max
//                    logit (raw)} for the 32-row tiles that can reach the bound
//   qn2  [H][4]      per head and 128-column block of q_abs: max over the
//                    virtual sequences of the block's squared norm (block 0
//                    also holds the q^R part)
constexpr int kDecList = 32;   // candidate tiles a split workgroup keeps per head
struct AbsorbedWs {
  size_t qabs, qlo, prefix, nflag, part_o, part_ml, dlb, dcnt, dent, qn2, total;
  int64_t slots;
};
inline AbsorbedWs absorbed_ws_layout(int heads, int batch, int tq) {
  AbsorbedWs w{};
  const int64_t bt = static_cast<int64_t>(batch) * tq;
  w.slots = kDecSplits + bt;
  size_t off = 0;
  w.qabs = off; off = align_up(off + static_cast<size_t>(bt) * heads * (kR + kS) * 2, 256);
  w.qlo = off; off = align_up(off + static_cast<size_t>(bt) * heads * kR * 2, 256);
  // prefix: bt + 1 row offsets of the virtual sequences, then the split
  // workgroups' kDecSplits + 1 row boundaries
  w.prefix = off; off = align_up(off + static_cast<size_t>(bt + 1 + kDecSplits + 1) * 8, 256);
  w.nflag = off; off = align_up(off + 4, 256);   // count of segments the fix-up kernel must redo
  w.part_o = off; off = align_up(off + static_cast<size_t>(w.slots) * heads * kR * 4, 256);
  w.part_ml = off; off = align_up(off + static_cast<size_t>(w.slots) * heads * 4 * 4, 256);
  w.dlb = off; off = align_up(off + static_cast<size_t>(kDecSplits) * heads * 4, 256);
  w.dcnt = off; off = align_up(off + static_cast<size_t>(kDecSplits) * heads * 4, 256);
  w.dent = off; off = align_up(off + static_cast<size_t>(kDecSplits) * heads * kDecList * 16, 256);
  w.qn2 = off; off = align_up(off + static_cast<size_t>(heads) * 4 * 4, 256);
  w.total = off;
  return w;
}

// Workspace of the bf16 expanded-cache decode: per (query, head, split of
// kExpSplitRows visible rows) the unnormalised output [V] and {max (log2
// units), sum}.
constexpr int kExpSplitRows = 2048;
struct ExpandedWs {
  size_t part_o, part_ml, total;
  int smax;   // splits per (query, head): ceil(cap / kExpSplitRows)
};
inline ExpandedWs expanded_ws_layout(int heads, int batch, int tq, int64_t cap) {
  ExpandedWs w{};
  w.smax = static_cast<int>((cap + kExpSplitRows - 1) / kExpSplitRows);
  const size_t items = static_cast<size_t>(batch) * tq * heads * w.smax;
  size_t off = 0;
  w.part_o = off; off = align_up(off + items * kV * 4, 256);
  w.part_ml = off; off = align_up(off + items * 2 * 4, 256);
  w.total = off;
  return w;
}

// Workspace of the bf16 whole layer: the projections' outputs and the norms'
// (bf16, row-major), then the prefill's own workspace.
constexpr int kGemmMaxProblems = 3;
struct LayerWs {
  size_t cq, ckv_raw, g, cqn, ckvn, ks, q, o, prefill, total;
};
inline LayerWs layer_ws_layout(int heads, int hidden, int q_rank, int64_t ntok, int nseq) {
  (void)hidden;
  LayerWs w{};
  const size_t T = static_cast<size_t>(ntok);
  size_t off = 0;
  w.cq = off; off = align_up(off + T * q_rank * 2, 256);
  w.ckv_raw = off; off = align_up(off + T * (kR + kS) * 2, 256);
  w.g = off; off = align_up(off + T * heads * kV * 2, 256);
  w.cqn = off; off = align_up(off + T * q_rank * 2, 256);
  w.ckvn = off; off = align_up(off + T * kR * 2, 256);
  w.ks = off; off = align_up(off + T * kS * 2, 256);
  w.q = off; off = align_up(off + T * heads * kD * 2, 256);
  w.o = off; off = align_up(off + T * heads * kV * 2, 256);
  w.prefill = off; off = align_up(off + prefill_ws_layout(heads, ntok, nseq).total, 256);
  w.total = off;
  return w;
}

// Workspace of the bf16 prefill backward (all O(T H)): [K^C | V] of every
// head, dO~ (bf16), {lse log2(e), D} per head and token, [dK^C | dV] (bf16) and
// its transpose, the transposed weight and latent, the per-head k^S
// gradients, the two work-item lists of the attention passes, and the
// split-K partials of the weight products.
struct BackwardWs {
  size_t kv, dot, lsed, dkv, dkvT, wT, ckvT, dksp, part, items_kv, items_q, count, total;
  int64_t items;   // capacity of each work-item list: ceil(T / 128) + nseq
  int split_c, split_w;   // K splits of dc^KV and dW
};
BackwardWs backward_ws_layout(int heads, int64_t ntok, int nseq);

// QK-norm variant: per-head RMSNorm of the queries over their N + S features,
// times a per-feature weight shared by the heads (w NULL: ones), the result
// rounded to the input dtype where it is formed. Off when `on` is false.
struct QNorm {
  const void* w = nullptr;
  float eps = 0.0f;
  bool on = false;
};

// ---- launchers (defined next to their kernels) ----

hipError_t launch_fill(float* p, int n, float v, hipStream_t st);

hipError_t launch_prefill_bf16(int heads, float scale, bool out_bf16,
                               const void* q, const void* ckv, const void* ks, const void* w_kv_b,
                               const void* gate, const int32_t* cu, int nseq, int64_t ntok,
                               void* out, float* lse, float* max_logit, bool init_max_logit, void* ws,
                               hipStream_t st, const QNorm& qn = QNorm{});

hipError_t launch_prefill_f32(int heads, int R, int S, int N, int V, float scale,
                              const float* q, const float* ckv, const float* ks, const float* w_kv_b,
                              const float* gate, const int32_t* cu, int nseq, int64_t ntok,
                              float* out, float* lse, float* max_logit, void* ws, hipStream_t st,
                              const QNorm& qn = QNorm{});

hipError_t launch_absorbed_bf16(int heads, float scale, bool out_bf16,
                                const void* q, const void* cache, int64_t cap, const int32_t* lens,
                                int batch, int tq, const void* w_kv_b, const void* gate, void* out,
                                float* max_logit, bool init_max_logit, void* ws, hipStream_t st,
                                const QNorm& qn = QNorm{});

hipError_t launch_expanded_bf16(int heads, float scale, bool out_bf16, const void* q, const void* kcache,
                                const void* vcache, int64_t cap, const int32_t* lens, int batch, int tq,
                                const void* gate, void* out, float* max_logit, void* ws, hipStream_t st);

// C = A B^T (bf16 operands, K-contiguous rows; fp32 accumulation; bf16 or
// fp32 C) for up to kGemmMaxProblems (B, C) pairs sharing A, batched over
// blockIdx.y with element strides sa, sb, sc. K a multiple of 128.
struct GemmSpec {
  const uint16_t* b;
  void* c;
  int64_t ldb, ldc, sb, sc;
  int n;
};
hipError_t launch_gemm_bf16(bool out_f32, const uint16_t* a, int64_t lda, int64_t sa, int m, int k, int batch,
                            int nprob, const GemmSpec* p, const char* name, hipStream_t st);
hipError_t launch_linear_bf16(const void* x, int64_t m, int k, const void* w, int n, void* y, hipStream_t st);
hipError_t launch_rms_norm_bf16(const void* x, int64_t rows, int n, const void* w, float eps, void* y,
                                hipStream_t st);
hipError_t launch_layer_bf16(int heads, float scale, int hidden, int q_rank, float eps, const void* x,
                             const void* w_dq, const void* g_q, const void* w_uq, const void* w_kv_a,
                             const void* g_kv, const void* w_kv_b, const void* w_g, const void* w_o,
                             const int32_t* cu, int nseq, int64_t ntok, void* out, float* max_logit,
                             bool init_max_logit, void* ws, hipStream_t st);

hipError_t launch_prefill_backward_bf16(int heads, float scale, const void* q, const void* ckv, const void* ks,
                                        const void* w_kv_b, const void* gate, const int32_t* cu, int nseq,
                                        int64_t ntok, const float* out, const float* lse, const float* dout,
                                        float* dq, float* dckv, float* dks, float* dw, float* dgate, void* ws,
                                        hipStream_t st);

hipError_t launch_absorbed_f32(int heads, int R, int S, int N, int V, float scale,
                               const float* q, const float* cache, int64_t cap, const int32_t* lens,
                               int batch, int tq, const float* w_kv_b, const float* gate, float* out,
                               float* max_logit, hipStream_t st, const QNorm& qn = QNorm{});

hipError_t launch_qk_clip(int heads, int S, int N, int V, bool bf16, void* w_q_b, int q_in, int R,
                          void* w_kv_b, const float* max_logit, float tau, uint8_t* clipped,
                          float* gamma, hipStream_t st);

}  // namespace mla
