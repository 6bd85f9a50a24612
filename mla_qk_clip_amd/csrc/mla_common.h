// Device helpers shared by the libmla kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D = A x B + C with A: 32x16 (lane l holds row l%32, k-slots 8*(l/32)..+7),
// B: 16x32 (lane l holds column l%32, the same k-slots) and C/D: 32x32 with
// lane l holding column l%32, rows 8*(i/4) + 4*(l/32) + i%4 for i = 0..15.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D = A x B + C with A: 16x32 (lane l holds row l%16, k-slots 8*(l/16)..+7),
// B: 32x16 (lane l holds column l%16, the same k-slots) and C/D: 16x16 with
// lane l holding column l%16, rows 4*(l/16) + i for i = 0..3.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Row index (within a 32x32 accumulator block) of accumulator element i in a lane of half g.
__device__ __forceinline__ int acc_row(int i, int g) { return ((i >> 2) << 3) + (g << 2) + (i & 3); }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round two floats to bf16 (nearest-even) and pack them (a in the low half).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}
__device__ __forceinline__ uint16_t f32_to_bf16(float a) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(a));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float sigmoidf_(float x) {
  // 1 / (1 + e^-x); e^-x overflows to +inf for very negative x, giving 0.
  return __builtin_amdgcn_rcpf(1.0f + fast_exp2(-x * kLog2e));
}

// Order-preserving float max through integer atomics: non-negative floats
// compare like signed ints, negative floats like unsigned ints in reverse.
// The slot must start at -inf (or any float); NaN inputs are not expected.
__device__ __forceinline__ void atomic_max_float(float* addr, float v) {
  if (v >= 0.0f) {
    atomicMax(reinterpret_cast<int*>(addr), __float_as_int(v));
  } else {
    atomicMin(reinterpret_cast<unsigned int*>(addr), __float_as_uint(v));
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Max / sum of a value and the same value in the lane 32 apart (one
// cross-half swap, no LDS traffic).
// max(a, b, c) with NaN propagation (IEEE maximum: no operand quieting needed)
__device__ __forceinline__ float fmax3_(float a, float b, float c) {
  return __builtin_elementwise_maximum(a, __builtin_elementwise_maximum(b, c));
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmax3_(v, __uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Compile-time loop: f(std::integral_constant<int, I>) for I = B .. E-1, so
// that register arrays are always indexed by constants.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void stg16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

// Position of key/row index p (within an aligned group of 16) in the layout
// the value-side MFMA operands are read from: the 4-element groups 1 and 2
// trade places, so that lane half 0 finds rows {0-3, 8-11} and half 1 finds
// rows {4-7, 12-15} as 8 consecutive elements, matching the rows it holds in
// the score accumulator.
__host__ __device__ constexpr int vperm16(int p) { return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1); }
// The same exchange applied inside every aligned group of 16.
__host__ __device__ constexpr int kperm(int n) { return (n & ~15) | vperm16(n & 15); }

// Wait until at most N vector-memory operations of this wave are outstanding
// (global loads, including the ones that write LDS directly).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Raw buffer resource over [base, base + bytes) (reads past the end return 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

// Buffer load of 16 bytes per lane (at byte offset voff + soff of the
// resource) straight into LDS: lane i's bytes land at lds + 16 i (lds must be
// the same for the whole wave).
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

// Copy 16 bytes per lane from global memory straight into LDS: lane i's
// bytes land at lds + 16 i (lds must be the same for the whole wave).
__device__ __forceinline__ void dma16(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

__global__ void fill_f32_kernel(float* p, int n, float v);

}  // namespace mla
