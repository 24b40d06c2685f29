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

// OCP e4m3 -> bf16 is exact (3 mantissa bits fit in 7, every e4m3 exponent
// fits bf16's range); v_cvt_scalef32_pk_bf16_fp8 converts two codes per call.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint2 c) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, 1.0f, false);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, 1.0f, true);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, 1.0f, false);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, 1.0f, true);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
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

// ---- wave64 primitives on DPP (VALU lane moves, no LDS round trip) ----------------
// DPP controls (GFX9): quad_perm 0x00-0xFF, row_shr:n 0x110+n, row_mirror 0x140,
// row_half_mirror 0x141, row_bcast:15 0x142, row_bcast:31 0x143. Lanes whose
// source is out of range or masked off read 0 (bound_ctrl).
template <int CTRL, int ROW_MASK = 0xF, int BANK_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, ROW_MASK, BANK_MASK, true));
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  uint32_t x = v;
  x += dpp_u32<0x111>(v);
  x += dpp_u32<0x112>(v);
  x += dpp_u32<0x113>(v);
  x += dpp_u32<0x114, 0xF, 0xE>(x);
  x += dpp_u32<0x118, 0xF, 0xC>(x);
  x += dpp_u32<0x142, 0xA, 0xF>(x);
  x += dpp_u32<0x143, 0xC, 0xF>(x);
  return x;
}

__device__ __forceinline__ uint32_t lane_value(uint32_t v, int lane) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), lane));
}

// Sum of the 8 lanes 8j..8j+7 that contain this lane, in every one of them.
__device__ __forceinline__ uint32_t octet_sum(uint32_t x) {
  x += dpp_u32<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_u32<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_u32<0x141>(x);  // row_half_mirror
  return x;
}

// Wave-uniform max / min / sum.
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
  x = max(x, dpp_u32<0xB1>(x));
  x = max(x, dpp_u32<0x4E>(x));
  x = max(x, dpp_u32<0x141>(x));
  x = max(x, dpp_u32<0x140>(x));
  return max(max(lane_value(x, 0), lane_value(x, 16)), max(lane_value(x, 32), lane_value(x, 48)));
}
__device__ __forceinline__ uint32_t wave_min(uint32_t x) {
  x = min(x, dpp_u32<0xB1>(x));
  x = min(x, dpp_u32<0x4E>(x));
  x = min(x, dpp_u32<0x141>(x));
  x = min(x, dpp_u32<0x140>(x));
  return min(min(lane_value(x, 0), lane_value(x, 16)), min(lane_value(x, 32), lane_value(x, 48)));
}
__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
  return lane_value(wave_incl_scan(x), 63);
}

}  // namespace dsa
