// Shared device helpers for the gfx950 kernels of libxattn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kNumXcd = 8;   // MI355X: workgroups are dispatched round-robin over 8 XCDs

// D(32x32 fp32) += A(32x16 bf16) * B(16x32 bf16).
// Lane l supplies A row (l % 32), B column (l % 32), and k = 8*(l/32) .. +7.
// Lane l receives D column (l % 32), rows 8*(v/4) + 4*(l/32) + (v%4), v < 16.
__device__ __forceinline__ f32x16_t mfma_32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __builtin_bit_cast(float, b << 16);
}

// Work-item id for block `bid` of a grid padded to a multiple of kNumXcd, so
// that consecutive work items run on the same XCD (and share its L2).
__device__ __forceinline__ int xcd_swizzle(int bid, int grid) {
  const int per = grid / kNumXcd;
  return (bid % kNumXcd) * per + bid / kNumXcd;
}

}  // namespace xattn
