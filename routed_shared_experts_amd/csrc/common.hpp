// Device helpers shared by the gfx950 kernels: number-format conversions, the
// fully specified float32 exp/sigmoid used for routing decisions, and
// wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ---- bfloat16 (stored as uint16_t bit patterns) ---------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
// Round-to-nearest-even; inputs are finite.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// ---- OCP e4m3fn -------------------------------------------------------------
// The hardware converter rounds to nearest even but turns values past 448 into
// NaN, so the input is saturated to +-448 first (RNE with saturation).
__device__ __forceinline__ uint32_t pack2_e4m3(float a, float b) {
  a = fminf(fmaxf(a, -448.0f), 448.0f);
  b = fminf(fmaxf(b, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  return pack2_e4m3(a, b) | (pack2_e4m3(c, d) << 16);
}

// ---- specified float32 exp / sigmoid -----------------------------------------
// Every step is one correctly rounded IEEE float32 operation (no contraction):
// clamp to [-80, 80]; n = rint(x * log2 e); Cody-Waite reduction with
// LN2_HI = 45426/2^16 (exact products for |n| < 256) and LN2_LO = ln2 - LN2_HI;
// degree-7 Taylor polynomial (coefficients 1/j!) by Horner with separate
// multiply and add; scale by 2^n.  sigmoid(x) = 1 / (1 + exp(-x)).
// The operators are written out here (not through helper functions) so that
// the contract(off) pragma covers every multiply and add: helpers defined
// elsewhere would carry their own contraction flags and fuse into FMAs.
__device__ __forceinline__ float spec_exp(float x) {
#pragma clang fp contract(off)
  const float kLog2e = 1.44269504088896340736f;
  const float kLn2Hi = 45426.0f / 65536.0f;
  const float kLn2Lo = (float)(0.6931471805599453 - 45426.0 / 65536.0);
  x = fminf(fmaxf(x, -80.0f), 80.0f);
  const float n = __builtin_rintf(x * kLog2e);
  const float t1 = n * kLn2Hi;
  const float t2 = n * kLn2Lo;
  const float r = (x - t1) - t2;
  float p = (float)(1.0 / 5040.0);
  p = p * r;
  p = p + (float)(1.0 / 720.0);
  p = p * r;
  p = p + (float)(1.0 / 120.0);
  p = p * r;
  p = p + (float)(1.0 / 24.0);
  p = p * r;
  p = p + (float)(1.0 / 6.0);
  p = p * r;
  p = p + 0.5f;
  p = p * r;
  p = p + 1.0f;
  p = p * r;
  p = p + 1.0f;
  return __builtin_ldexpf(p, (int)n);
}
__device__ __forceinline__ float spec_sigmoid(float x) {
#pragma clang fp contract(off)
  const float d = 1.0f + spec_exp(-x);
  return 1.0f / d;  // correctly rounded fp32 division (HIP default)
}

// SiLU(g) * u for the stage-1 epilogue (ordinary accuracy is enough here).
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}
// act(g) * u: act = 0 SiLU; act = 1 GELU in its tanh form, written through
// 1 + tanh(z) = 2 sigmoid(2 z): g * sigmoid(2 sqrt(2/pi) (g + 0.044715 g^3)).
__device__ __forceinline__ float act_mul(float g, float u, int act) {
  if (act == 1) {
    const float z = g * (1.5957691216057308f + 0.07135481627159537f * (g * g));
    return g / (1.0f + __expf(-z)) * u;
  }
  return silu_mul(g, u);
}
// Bias entry i; without a bias (or past the valid width) -0, which adds to
// any value, signed zeros included, without changing it.
__device__ __forceinline__ float bias_at(const float* b, int i, int width = 0x7FFFFFFF) {
  return (b && i < width) ? b[i] : -0.0f;
}
// The epilogue of the register-heavy kernels, specialised: EPI = false is
// the plain SiLU-mul with no bias (the common case, no extra registers);
// EPI = true reads the biases and the activation choice.
template <bool EPI>
__device__ __forceinline__ float epi_bias(const float* b, int i, int width = 0x7FFFFFFF) {
  if constexpr (EPI) return bias_at(b, i, width);
  else return -0.0f;
}
template <bool EPI>
__device__ __forceinline__ float epi_act(float g, float u, int act) {
  if constexpr (EPI) return act_mul(g, u, act);
  else return silu_mul(g, u);
}

// ---- wave64 reductions --------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// ---- wave64 reductions through DPP (no LDS round trips) ----------------------
// row_shr:1,2,4,8 leave each row's total in its lane 15; row_bcast:15 and
// row_bcast:31 carry rows 0-2 into row 3, so lane 63 ends with the wave total,
// which readlane makes uniform.  Lanes with no DPP source keep their own value
// (max) or add zero (sum).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xF, false);
}
__device__ __forceinline__ uint32_t dpp_wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0x111, 0xF>(v, v));
  v = max(v, dpp_u32<0x112, 0xF>(v, v));
  v = max(v, dpp_u32<0x114, 0xF>(v, v));
  v = max(v, dpp_u32<0x118, 0xF>(v, v));
  v = max(v, dpp_u32<0x142, 0xA>(v, v));
  v = max(v, dpp_u32<0x143, 0xC>(v, v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ float dpp_wave_sum(float v) {
  v += __uint_as_float(dpp_u32<0x111, 0xF>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp_u32<0x112, 0xF>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp_u32<0x114, 0xF>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp_u32<0x118, 0xF>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp_u32<0x142, 0xA>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp_u32<0x143, 0xC>(0u, __float_as_uint(v)));
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 63));
}
// Maximum of 64-bit keys (hi, lo) over the wave: the largest hi, then the
// largest lo among the lanes holding it.  Returns the key, uniform.
__device__ __forceinline__ uint64_t dpp_wave_max_key(uint64_t k) {
  const uint32_t hi = (uint32_t)(k >> 32), lo = (uint32_t)k;
  const uint32_t mh = dpp_wave_max_u32(hi);
  const uint32_t ml = dpp_wave_max_u32(hi == mh ? lo : 0u);
  return ((uint64_t)mh << 32) | ml;
}

// Make this wave's LDS writes visible to its other lanes before they read.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  __builtin_amdgcn_wave_barrier();
}

// Order-preserving map of a float to uint32 (larger float -> larger key);
// -0 is folded onto +0 so that equal values tie.
__device__ __forceinline__ uint32_t float_key(float f) {
  f = f + 0.0f;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace moe
