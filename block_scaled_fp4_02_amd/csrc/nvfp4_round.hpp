// NVFP4 rounding steps shared by the quantiser and the fused SwiGLU + NVFP4 GEMM epilogue.
// Reading of the open steps (format: "Cracking the SM120 Shared Memory Ceiling", section
// "The Shared Memory Calculation"): block scale s = e4m3_rne(min(amax_b / (6 g), 448)),
// element code sign(x) | e2m1_rne(min(|x| / (s g), 6)) (0 / 0, a zero block or element over
// an underflowed g or s g, counts as 0), every step one correctly rounded
// binary32 operation in this order -- callers compile these with contraction off.
#pragma once

#include <stdint.h>

namespace moe {

// Nearest E4M3FN code to t in [0, 448], ties to the even code.
__device__ __forceinline__ uint32_t e4m3_rne(float t) {
  if (t < 0.015625f) return static_cast<uint32_t>(rintf(t * 512.0f));  // multiples of 2^-9
  uint32_t u = __float_as_uint(t);
  u += 0x7ffffu + ((u >> 20) & 1u);  // round the 23-bit mantissa to 3 bits, ties to even
  return (u >> 20) - (120u << 3);    // rebias the exponent from 127 to 7
}

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  if (c < 8u) return static_cast<float>(c) * 0.001953125f;  // subnormal: c * 2^-9
  return __uint_as_float((((c >> 3) + 120u) << 23) | ((c & 7u) << 20));
}

// E2M1 magnitude code for u in [0, 6], ties to the even code.  Below 1 the E2M1 values are
// the multiples of 0.5 (code = 2u rounded to nearest even); from 1 up they have one mantissa
// bit, so the binary32 mantissa is rounded to one bit and the exponent rebiased (127 -> 1).
__device__ __forceinline__ uint32_t e2m1_rne(float u) {
  if (u < 1.0f) return static_cast<uint32_t>(rintf(u * 2.0f));
  uint32_t b = __float_as_uint(u);
  b += 0x1fffffu + ((b >> 22) & 1u);
  return (b >> 22) - (126u << 1);
}

// Correctly rounded binary32 quotients a / b of one block by one divisor b = s * g, from a
// single correctly rounded reciprocal y = 1 / b and fma corrections.  q0 = a * y can be a
// little more than one ulp from a / b; one correction q1 = q0 + (a - q0 b) y makes it
// faithful (within one ulp), the remainder r1 = a - q1 b is then exact as one fma, and
// q1 + r1 y rounded once is the correctly rounded quotient (Markstein's theorem on division
// by fused multiply-add, which needs y correctly rounded and q1 faithful; Muller et al.,
// Handbook of Floating-Point Arithmetic, the chapter on algorithms using the fma).  The
// theorem needs every step clear of underflow and overflow, so the form applies only when
// b lies well inside the normal range and the block maximum over b stays far below
// overflow; otherwise (`fast` false, which covers b = 0) the caller divides each element.
// Quotients small enough to underflow round to the E2M1 code 0 either way.
struct BlockDivisor {
  float b, y;
  bool fast;
};

__device__ __forceinline__ BlockDivisor block_divisor(float b, float amax) {
  BlockDivisor d;
  d.b = b;
  d.y = 1.0f / b;
  d.fast = b >= 0x1p-100f && b <= 0x1p100f && amax * d.y < 0x1p100f;
  return d;
}

__device__ __forceinline__ float block_quotient(float a, const BlockDivisor &d) {
  const float q0 = a * d.y;
  const float r0 = __builtin_fmaf(-q0, d.b, a);
  const float q1 = __builtin_fmaf(r0, d.y, q0);  // faithful
  const float r1 = __builtin_fmaf(-q1, d.b, a);  // exact
  return __builtin_fmaf(r1, d.y, q1);
}

// E2M1 codes of eight non-negative binary32 values, two per hardware conversion, packed
// low nibble first.  With a unit scale the conversion rounds to nearest even and saturates
// at 6, and equals e2m1_rne(min(u, 6)) for every non-negative binary32 u (every such bit
// pattern, +inf included, checked on gfx950).
__device__ __forceinline__ uint32_t e2m1_pack8(const float (&u)[8]) {
  uint32_t w = 0u;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, u[0], u[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, u[2], u[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, u[4], u[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, u[6], u[7], 1.0f, 3);
  return w;
}

__device__ __forceinline__ uint32_t e2m1_pack4(const float (&u)[4]) {
  uint32_t w = 0u;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, u[0], u[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, u[2], u[3], 1.0f, 1);
  return w;
}

}  // namespace moe
