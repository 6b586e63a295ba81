// Device helpers shared by the gfx950 attention kernels: MFMA wrappers, bf16
// packing, cross-half reductions, exp2 variants and LDS swizzles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Conditional rescale threshold in log2 units: the accumulator is rescaled
// only when a row max grows by more than log2(256) = 8, so unnormalised
// probabilities stay below 2^8 (hotelren summary, section 3.3).
constexpr float kTau = 8.0f;

// 32x32x16 bf16 MFMA with fp32 accumulate (gfx950).  Operand layout per lane l:
// A holds row m = l % 32 and 8 consecutive k slots of half l / 32; B holds
// column n = l % 32 and the same k slots; the 16 accumulator registers hold
// column n = l % 32 and rows m = 8 * (r / 4) + 4 * (l / 32) + r % 4.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }

// Two fp32 -> packed bf16x2 (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b16) {
  return __builtin_bit_cast(float, b16 << 16);
}

// Value of the same register in lane l ^ 32 (the other half of the wave).
__device__ __forceinline__ float xhalf(float v) { return __shfl_xor(v, 32, 64); }

// Hardware exp2 (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// exp2 on FMA/ALU units only: x = n + f with n = floor(x), f in [0, 1),
// 2^f ~ 1 + f (c1 + f (c2 + f c3)), and n added to the exponent field
// (hotelren summary, section 3.2; danialwang explainer, 巧招一).  The
// coefficients are a minimax fit of the relative error with p(0) = 1 exactly
// (fit_exp2_poly.py); the fit's bound is 8.6e-5, below bf16's 2^-9.  Inputs
// below -127 give 0 (so a masked -inf gives exactly 0).
constexpr float kExp2C1 = 0.695117295f;
constexpr float kExp2C2 = 0.227643535f;
constexpr float kExp2C3 = 0.0770680308f;
__device__ __forceinline__ float exp2_poly(float x) {
  const float xc = __builtin_fmaxf(x, -127.0f);
  const float n = __builtin_floorf(xc);
  const float f = xc - n;
  float p = __builtin_fmaf(f, kExp2C3, kExp2C2);
  p = __builtin_fmaf(f, p, kExp2C1);
  p = __builtin_fmaf(f, p, 1.0f);
  const int32_t bits = __builtin_bit_cast(int32_t, p) + ((int32_t)n << 23);
  return x < -127.0f ? 0.0f : __builtin_bit_cast(float, bits);
}

}  // namespace fa
