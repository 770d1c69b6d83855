// Shared device-side types and helpers for the gfx950 DiT kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

typedef uint16_t bf16_t;  // bfloat16 bit pattern as stored in HBM

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Four fp32 -> four bf16 (round to nearest even, the hardware conversion).
__device__ __forceinline__ u32x2 pack_bf16x4(f32x4 v) {
  bf16x4 b = __builtin_convertvector(v, bf16x4);
  return __builtin_bit_cast(u32x2, b);
}

__device__ __forceinline__ bf16x8 pack_bf16x8(f32x8 v) {
  return __builtin_convertvector(v, bf16x8);
}

__device__ __forceinline__ float silu_f(float v) {
  return v / (1.0f + __expf(-v));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Sum across aligned groups of `width` lanes (width a power of two <= 64).
template <int width>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = width / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// max / sum of x over lanes l and l ^ 32 (gfx950 v_permlane32_swap, no LDS)
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t clamp_u32(int64_t v) {
  return v > 0xFFFFFFFFll ? 0xFFFFFFFFu : static_cast<uint32_t>(v);
}

// Buffer resource for raw (unswizzled) buffer loads; reads at byte offsets
// >= `bytes` return zero. Every input is made wave-uniform so the descriptor
// lives in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
  void* base = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)n, 0x00020000);
}

// Workgroups are handed to the 8 XCDs round-robin by launch index. Remap the
// launch index so that consecutive logical tiles run on the same XCD (and so
// share its L2): XCD x receives logical tiles [start_x, start_x + count_x).
__device__ __forceinline__ int xcd_remap(int wg, int n_wg) {
  const int x = wg & 7, k = wg >> 3;
  const int q = n_wg >> 3, r = n_wg & 7;
  return (x < r) ? x * (q + 1) + k : r * (q + 1) + (x - r) * q + k;
}

}  // namespace dit
