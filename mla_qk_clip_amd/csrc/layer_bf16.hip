// The whole gated MLA attention layer in bf16 ("Kimi K3 · Gated MLA ·
// OpenModelAtlas": the 20-step equation list and the KimiMLAAttention
// excerpts): every projection is nn.Linear without bias, y = x W^T with
// W = weight [out, in]:
//   c^Q = x W_DQ  (q_a_proj),  c^Q^ = RMSNorm(c^Q),  q = c^Q^ W_UQ  (q_b_proj),
//   [c^KV | k^S] = x W_DKV  (kv_a_proj_with_mqa),  c^KV^ = RMSNorm(c^KV),
//   g = x W_g  (g_proj),  o = sigma(g) . attention  (the prefill kernels),
//   Delta = o W_O  (o_proj).
//
// Kernels:
//  - gemm_nt_kernel: C = A B^T for up to three B/C pairs that share A (the
//    three projections of x run as one launch). 256 x 256 output tiles, 8
//    waves (wave w: rows 64 (w & 3) .., columns 128 (w >> 2) ..), K (a
//    multiple of 128) in steps of 64 through two LDS slots filled by buffer loads straight to LDS one
//    step ahead: every copy instruction moves 8 whole 128-byte row segments,
//    and the tile layout (unit (r, c) at 64 (r/8) + 8 (r%8) + (c ^ (r/2)%8))
//    keeps the fragment reads free of bank conflicts. Rows past M or N read
//    zeros (buffer range check). The products are formed transposed (C^T =
//    B A^T: accumulator lane = output row), and a cross-half lane swap turns
//    each lane's four 4-column runs into two 8-column runs: 16-byte stores
//    of the row-major bf16 output.
//  - rmsnorm_kernel: one wave per row, fp32 sum of squares, bf16 output; the
//    latent job also copies the k^S columns out of [c^KV | k^S].
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "mla_common.h"
#include "mla_internal.h"
#include "timing.h"

namespace mla {

namespace {

constexpr int kGmT = 256;            // output tile rows and columns
constexpr int kGmThreads = 512;
constexpr int kGmUnits = kGmT * 8;   // 16-byte units of one operand slot (256 rows x 128 bytes)

struct GemmProblem {
  const uint16_t* b;
  void* c;          // bf16 or fp32, row-major
  int64_t ldb, ldc;
  int64_t sb, sc;   // batch strides (elements) of B and C
  int n;       // columns of C (rows of B)
  int tile0;   // first column tile of this problem in the combined tile space
};
struct GemmArgs {
  const uint16_t* a;
  int64_t lda, sa;   // row stride and batch stride (elements) of A
  int m, k;
  int nprob, mtiles, ntiles;
  GemmProblem p[kGemmMaxProblems];
};

// blockIdx.y is the batch index (a separate A, B and C per batch entry).
// kOutF32: fp32 C, else bf16.
template <bool kOutF32>
__global__ void __launch_bounds__(kGmThreads) gemm_nt_kernel(GemmArgs args) {
  __shared__ uint4 As0[kGmUnits], As1[kGmUnits];
  __shared__ uint4 Bs0[kGmUnits], Bs1[kGmUnits];

  // items are dealt to the XCDs in contiguous ranges (block b runs on XCD b % 8)
  const int total = args.mtiles * args.ntiles;
  const int per_xcd = (total + 7) >> 3;
  const int item = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (item >= total) return;
  // groups of 8 row tiles x all column tiles, row tile fastest inside a group:
  // an XCD's 32 concurrent workgroups cover 8 row tiles x 4 column tiles
  constexpr int kGroupM = 8;
  const int group = item / (kGroupM * args.ntiles);
  const int first_m = group * kGroupM;
  const int gm = min(args.mtiles - first_m, kGroupM);
  const int in_group = item - group * kGroupM * args.ntiles;
  const int mt = first_m + in_group % gm;
  const int nt = in_group / gm;
  // this tile's problem (selected field by field: indexing the argument array
  // would copy it to private memory)
  const bool p1 = args.nprob > 1 && nt >= args.p[1].tile0;
  const bool p2 = args.nprob > 2 && nt >= args.p[2].tile0;
  const int64_t bz = blockIdx.y;
  const GemmProblem P{(p2 ? args.p[2].b : p1 ? args.p[1].b : args.p[0].b) +
                          bz * (p2 ? args.p[2].sb : p1 ? args.p[1].sb : args.p[0].sb),
                      p2 ? args.p[2].c : p1 ? args.p[1].c : args.p[0].c,
                      p2 ? args.p[2].ldb : p1 ? args.p[1].ldb : args.p[0].ldb,
                      p2 ? args.p[2].ldc : p1 ? args.p[1].ldc : args.p[0].ldc,
                      0,
                      bz * (p2 ? args.p[2].sc : p1 ? args.p[1].sc : args.p[0].sc),
                      p2 ? args.p[2].n : p1 ? args.p[1].n : args.p[0].n,
                      p2 ? args.p[2].tile0 : p1 ? args.p[1].tile0 : args.p[0].tile0};
  const uint16_t* a_base = args.a + bz * args.sa;
  const int m0 = mt * kGmT, n0 = (nt - P.tile0) * kGmT;
  const int rows_a = min(kGmT, args.m - m0), rows_b = min(kGmT, P.n - n0);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int wm = wave & 3;

  // staging: copy q of wave w covers tile rows 8 (4 w + q) .. +7; lane i takes
  // row 8 (4 w + q) + i / 8 and k-unit (i % 8) ^ ((row / 2) % 8)
  const auto rs_a = make_rsrc(a_base + static_cast<int64_t>(m0) * args.lda,
                              static_cast<uint32_t>(rows_a * args.lda * 2));
  const auto rs_b = make_rsrc(P.b + static_cast<int64_t>(n0) * P.ldb, static_cast<uint32_t>(rows_b * P.ldb * 2));
  uint32_t voff_a[4], voff_b[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 8 * (4 * wave + q) + (lane >> 3), c = (lane & 7) ^ ((r >> 1) & 7);
    voff_a[q] = static_cast<uint32_t>(r * args.lda * 2 + 16 * c);   // rows past the matrix: past the range, zeros
    voff_b[q] = static_cast<uint32_t>(r * P.ldb * 2 + 16 * c);
  }
  auto issue = [&](uint4* ad, uint4* bd, int st) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      dma16_buf(rs_a, voff_a[q], 128 * st, ad + 64 * (4 * wave + q));
      dma16_buf(rs_b, voff_b[q], 128 * st, bd + 64 * (4 * wave + q));
    }
  };
  // copy c (0..7) of a step: A block c / 2 or B block c / 2
  auto issue_one = [&](uint4* ad, uint4* bd, int st, int c) {
    const int q = c >> 1;
    if (c & 1) dma16_buf(rs_b, voff_b[q], 128 * st, bd + 64 * (4 * wave + q));
    else dma16_buf(rs_a, voff_a[q], 128 * st, ad + 64 * (4 * wave + q));
  };
  // Fragment reads: rows r0 .. r0+31 (r0 a multiple of 32), k-units 2 kh + g.
  // Unit 64 (r/8) + 8 (r%8) + (c ^ (r/2)%8) splits into the wave-uniform
  // 8 r0 and a per-lane part that depends on kh only.
  int lp[4];
#pragma unroll
  for (int kh = 0; kh < 4; ++kh) lp[kh] = 64 * (l32 >> 3) + 8 * (l32 & 7) + ((2 * kh + g) ^ ((l32 >> 1) & 7));
  auto frag = [&](const uint4* t, int r0, int kh) { return as_bf16x8(t[8 * r0 + lp[kh]]); };

  // Each half of the waves (column blocks wn = 0, 1) runs its own copy of the
  // loop, so that the fragment addresses fold into immediate offsets.
  auto run = [&](auto WN) {
    constexpr int wn = decltype(WN)::value;
    // acc[2 fb + kb]: column block fb (4 x 32 of the wave's 128), row block kb (2 x 32 of its 64)
    f32x16 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = f32x16{};
    // one k-step; copy c of the next step goes out after MFMA 4 c + 1 + 2 wn
    // (the two waves of a SIMD alternate their copy stalls)
    auto step = [&](const uint4* as, const uint4* bs, auto&& cp) {
#pragma unroll
      for (int kh = 0; kh < 4; ++kh) {
        bf16x8 af[2], bf[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) af[kb] = frag(as, 64 * wm + 32 * kb, kh);
#pragma unroll
        for (int fb = 0; fb < 4; ++fb) bf[fb] = frag(bs, 128 * wn + 32 * fb, kh);
#pragma unroll
        for (int fb = 0; fb < 4; ++fb)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            acc[2 * fb + kb] = mfma32(bf[fb], af[kb], acc[2 * fb + kb]);
            const int m = 8 * kh + 2 * fb + kb;
            if (m < 16 && (m & 1) == wn) {   // copies in the first half of the step: they land before its end
              __builtin_amdgcn_sched_barrier(0);
              cp(m >> 1);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
      }
    };
    auto none = [](int) {};
    const int nsteps = args.k / 64;
    issue(As0, Bs0, 0);
    wait_vmcnt<0>();
    __syncthreads();
    int st = 0;
    for (; st + 2 < nsteps; st += 2) {   // steps st (slot 0) and st + 1 (slot 1), each copying the next
      // (slot 1 was last read by step st - 1)
      step(As0, Bs0, [&](int c) { issue_one(As1, Bs1, st + 1, c); });
      wait_vmcnt<0>();
      __syncthreads();
      step(As1, Bs1, [&](int c) { issue_one(As0, Bs0, st + 2, c); });
      wait_vmcnt<0>();
      __syncthreads();
    }
    // the last two steps (K is a multiple of 128)
    step(As0, Bs0, [&](int c) { issue_one(As1, Bs1, st + 1, c); });
    wait_vmcnt<0>();
    __syncthreads();
    step(As1, Bs1, none);

    // ---- store: lane = output row l32 of the row block; element i of a tile is
    // column 8 (i / 4) + 4 g + i % 4 of the column block. Lanes l and l + 32 swap
    // runs so that each holds 8 consecutive columns (two 16-byte stores per tile).
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int m = m0 + 64 * wm + 32 * kb + l32;
#pragma unroll
      for (int fb = 0; fb < 4; ++fb) {
        const f32x16 a = acc[2 * fb + kb];
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {   // runs 2 pr (kept by g = 0) and 2 pr + 1 (kept by g = 1)
          const int n = n0 + 128 * wn + 32 * fb + 16 * pr + 8 * g;
          if constexpr (kOutF32) {
            uint32_t x[4], y[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(a[8 * pr + e]),
                                                               __float_as_uint(a[8 * pr + 4 + e]), false, false);
              x[e] = sw[0];
              y[e] = sw[1];
            }
            if (m < args.m && n < P.n) {
              float* dst = static_cast<float*>(P.c) + P.sc + static_cast<int64_t>(m) * P.ldc + n;
              stg16(dst, make_uint4(x[0], x[1], x[2], x[3]));
              stg16(dst + 4, make_uint4(y[0], y[1], y[2], y[3]));
            }
          } else {
            uint32_t x[2], y[2];
#pragma unroll
            for (int w = 0; w < 2; ++w) {
              const uint32_t lo = pack_bf16x2(a[8 * pr + 2 * w], a[8 * pr + 2 * w + 1]);
              const uint32_t hi = pack_bf16x2(a[8 * pr + 4 + 2 * w], a[8 * pr + 4 + 2 * w + 1]);
              const auto sw = __builtin_amdgcn_permlane32_swap(lo, hi, false, false);
              x[w] = sw[0];
              y[w] = sw[1];
            }
            if (m < args.m && n < P.n)
              stg16(static_cast<uint16_t*>(P.c) + P.sc + static_cast<int64_t>(m) * P.ldc + n,
                    make_uint4(x[0], x[1], y[0], y[1]));
          }
        }
      }

    }
  };
  if (wave < 4) run(std::integral_constant<int, 0>{});
  else run(std::integral_constant<int, 1>{});
}

// One wave per row. Job 0: y0 = RMSNorm(x0) (width n0). Job 1: y1 =
// RMSNorm(first n1 columns of x1) and ytail = its next ntail columns.
struct NormJob {
  const uint16_t* x;
  const uint16_t* w;
  uint16_t* y;
  uint16_t* ytail;
  int64_t ldx;
  int n, ntail;
};

__global__ void __launch_bounds__(256) rmsnorm_kernel(NormJob j0, NormJob j1, int64_t rows, float eps) {
  const NormJob& J = blockIdx.y == 0 ? j0 : j1;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const uint16_t* xr = J.x + row * J.ldx;
  const int units = J.n / 8;
  constexpr int kMaxU = 4;   // up to 4 x 64 units (2048 features) per row
  uint4 v[kMaxU];
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < kMaxU; ++k) {
    const int u = lane + 64 * k;
    v[k] = u < units ? ldg16(xr + 8 * u) : make_uint4(0, 0, 0, 0);
    const uint32_t* p = &v[k].x;
#pragma unroll
    for (int e = 0; e < 4; ++e) s = fmaf(bf16lo(p[e]), bf16lo(p[e]), fmaf(bf16hi(p[e]), bf16hi(p[e]), s));
  }
  s = wave_sum(s);
  const float r = 1.0f / sqrtf(s / static_cast<float>(J.n) + eps);
  uint16_t* yr = J.y + row * J.n;
#pragma unroll
  for (int k = 0; k < kMaxU; ++k) {
    const int u = lane + 64 * k;
    if (u >= units) continue;
    const uint4 wv = ldg16(J.w + 8 * u);
    const uint32_t* p = &v[k].x;
    const uint32_t* q = &wv.x;
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = pack_bf16x2(bf16lo(p[e]) * r * bf16lo(q[e]), bf16hi(p[e]) * r * bf16hi(q[e]));
    stg16(yr + 8 * u, make_uint4(o[0], o[1], o[2], o[3]));
  }
  if (J.ytail && lane < J.ntail / 8) stg16(J.ytail + row * J.ntail + 8 * lane, ldg16(xr + J.n + 8 * lane));
}

}  // namespace

hipError_t launch_gemm_bf16(bool out_f32, const uint16_t* a, int64_t lda, int64_t sa, int m, int k, int batch,
                            int nprob, const GemmSpec* p, const char* name, hipStream_t st) {
  GemmArgs args{};
  args.a = a;
  args.lda = lda;
  args.sa = sa;
  args.m = m;
  args.k = k;
  args.nprob = nprob;
  args.mtiles = (m + kGmT - 1) / kGmT;
  int tiles = 0;
  for (int i = 0; i < nprob; ++i) {
    args.p[i] = GemmProblem{p[i].b, p[i].c, p[i].ldb, p[i].ldc, p[i].sb, p[i].sc, p[i].n, tiles};
    tiles += (p[i].n + kGmT - 1) / kGmT;
  }
  args.ntiles = tiles;
  const int total = args.mtiles * tiles;
  if (total == 0 || batch == 0) return hipSuccess;
  const dim3 grid(((total + 7) / 8) * 8, batch);
  TimedScope ts_(name, st);
  if (out_f32) hipLaunchKernelGGL(gemm_nt_kernel<true>, grid, dim3(kGmThreads), 0, st, args);
  else hipLaunchKernelGGL(gemm_nt_kernel<false>, grid, dim3(kGmThreads), 0, st, args);
  return hipGetLastError();
}


hipError_t launch_linear_bf16(const void* x, int64_t m, int k, const void* w, int n, void* y, hipStream_t st) {
  const GemmSpec p{static_cast<const uint16_t*>(w), y, k, n, 0, 0, n};
  return launch_gemm_bf16(false, static_cast<const uint16_t*>(x), k, 0, static_cast<int>(m), k, 1, 1, &p, "linear", st);
}

hipError_t launch_rms_norm_bf16(const void* x, int64_t rows, int n, const void* w, float eps, void* y,
                                hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const NormJob j{static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w), static_cast<uint16_t*>(y),
                  nullptr, n, n, 0};
  TimedScope ts_("rms_norm", st);
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(static_cast<unsigned>((rows + 3) / 4), 1), dim3(256), 0, st, j, j, rows,
                     eps);
  return hipGetLastError();
}

hipError_t launch_layer_bf16(int heads, float scale, int hidden, int q_rank, float eps, const void* x,
                             const void* w_dq, const void* g_q, const void* w_uq, const void* w_kv_a,
                             const void* g_kv, const void* w_kv_b, const void* w_g, const void* w_o,
                             const int32_t* cu, int nseq, int64_t ntok, void* out, float* max_logit,
                             bool init_max_logit, void* ws, hipStream_t st) {
  const LayerWs L = layer_ws_layout(heads, hidden, q_rank, ntok, nseq);
  char* base = static_cast<char*>(ws);
  auto buf = [&](size_t off) { return reinterpret_cast<uint16_t*>(base + off); };
  const int m = static_cast<int>(ntok);
  const int HV = heads * kV, HD = heads * kD, RS = kR + kS;
  hipError_t e;
  {  // c^Q, [c^KV | k^S] and g from x: one launch
    const GemmSpec p[3] = {{static_cast<const uint16_t*>(w_dq), buf(L.cq), hidden, q_rank, 0, 0, q_rank},
                           {static_cast<const uint16_t*>(w_kv_a), buf(L.ckv_raw), hidden, RS, 0, 0, RS},
                           {static_cast<const uint16_t*>(w_g), buf(L.g), hidden, HV, 0, 0, HV}};
    e = launch_gemm_bf16(false, static_cast<const uint16_t*>(x), hidden, 0, m, hidden, 1, 3, p, "layer_proj_x", st);
    if (e != hipSuccess) return e;
  }
  {
    const NormJob jq{buf(L.cq), static_cast<const uint16_t*>(g_q), buf(L.cqn), nullptr, q_rank, q_rank, 0};
    const NormJob jkv{buf(L.ckv_raw), static_cast<const uint16_t*>(g_kv), buf(L.ckvn), buf(L.ks), RS, kR, kS};
    TimedScope ts_("layer_norm", st);
    hipLaunchKernelGGL(rmsnorm_kernel, dim3(static_cast<unsigned>((ntok + 3) / 4), 2), dim3(256), 0, st, jq, jkv,
                       ntok, eps);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    const GemmSpec p{static_cast<const uint16_t*>(w_uq), buf(L.q), q_rank, HD, 0, 0, HD};
    e = launch_gemm_bf16(false, buf(L.cqn), q_rank, 0, m, q_rank, 1, 1, &p, "layer_proj_q", st);
    if (e != hipSuccess) return e;
  }
  e = launch_prefill_bf16(heads, scale, true, buf(L.q), buf(L.ckvn), buf(L.ks), w_kv_b, buf(L.g), cu, nseq, ntok,
                          buf(L.o), nullptr, max_logit, init_max_logit, base + L.prefill, st);
  if (e != hipSuccess) return e;
  {
    const GemmSpec p{static_cast<const uint16_t*>(w_o), out, HV, hidden, 0, 0, hidden};
    e = launch_gemm_bf16(false, buf(L.o), HV, 0, m, HV, 1, 1, &p, "layer_proj_o", st);
  }
  return e;
}

}  // namespace mla
