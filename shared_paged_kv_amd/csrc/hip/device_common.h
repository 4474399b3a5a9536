// Device helpers for the gfx950 kernels: bf16 bit handling, DPP lane
// reductions and the RoPE pair rotation.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvp {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// a.x*b.x + a.y*b.y + c for bf16 pairs packed in 32-bit words (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// DPP controls (gfx9 encoding)
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;      // lane i <-> 15-i within 16

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N lanes (N in 2, 4, 8, 16); every lane gets the sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<kDppXor1>(x);
  if constexpr (N >= 4) x += dpp<kDppXor2>(x);
  if constexpr (N >= 8) x += dpp<kDppHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kDppMirror>(x);
  return x;
}

// Rotation of one rotate-half pair (x1 at i, x2 at i + d/2) by angle delta*theta_i,
// theta_i = base^(-2i/d); the angle is formed in float64, cos and sin are rounded
// to float32, the rotation is done in float32.
__device__ __forceinline__ double rope_theta(int i, int d, float base) {
  return pow((double)base, -2.0 * (double)i / (double)d);
}

__device__ __forceinline__ void rope_cs_theta(int32_t delta, double th, float* c, float* s) {
  double a = (double)delta * th;
  double sd, cd;
  sincos(a, &sd, &cd);
  *c = (float)cd;
  *s = (float)sd;
}

__device__ __forceinline__ void rope_cs(int32_t delta, int i, int d, float base, float* c, float* s) {
  rope_cs_theta(delta, rope_theta(i, d, base), c, s);
}

// The fused multiply-adds are spelled out so that every kernel rounds a rotation
// the same way (an inferred contraction could pick either product).
__device__ __forceinline__ void rope_apply(float x1, float x2, float c, float s, float* y1, float* y2) {
  *y1 = fmaf(x1, c, -(x2 * s));
  *y2 = fmaf(x2, c, x1 * s);
}

}  // namespace kvp
