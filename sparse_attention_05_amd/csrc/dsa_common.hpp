// Device-side building blocks shared by the DSA kernels (gfx950 / CDNA4).
//
// MFMA operand layout used throughout (v_mfma_f32_16x16x32_bf16 and
// v_mfma_f32_16x16x4_f32, wave64): lane l = n + 16*g (n = l % 16, g = l / 16)
//   A (16 x K): lane holds row m = n, K-slots of group g
//   B (K x 16): lane holds column n, K-slots of group g
//   C (16 x 16): lane holds column n, rows 4*g + i for i = 0..3
// The contraction is a plain sum over K, so any bijection between K-slots
// and the contracted index works as long as A and B use the same one; the
// kernels pick bijections that make each lane's slots contiguous in memory.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

constexpr int kLatentDim = 576;
constexpr int kValueDim = 512;
constexpr int kMaxTopk = 2048;

enum : int { kF32 = 0, kBF16 = 1, kFP8 = 2 };

// One K=32 step of a 16x16 fp32-accumulating product.
// bf16: one v_mfma_f32_16x16x32_bf16 on 8 slots per lane.
__device__ __forceinline__ f32x4 mfma_k32(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// fp32 operands: 8 values per lane = 8 v_mfma_f32_16x16x4_f32, element j of
// every lane forming the 4 K-slots of instruction j.
struct f32x8 {
  float v[8];
};
__device__ __forceinline__ f32x4 mfma_k32(const f32x8& a, const f32x8& b, f32x4 c) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], c, 0, 0, 0);
  return c;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Order-preserving image of an fp32 score: a > b (IEEE) <=> key(a) > key(b)
// for non-NaN values, with -0.0 mapped to the key of +0.0.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <typename T>
__device__ __forceinline__ T wave_shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, 64);
}

}  // namespace dsa
