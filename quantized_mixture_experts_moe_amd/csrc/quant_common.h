// Per-row requantization of the intermediate h (shared by the requant kernel
// and the resident stage 2, which quantizes while it copies h rows to LDS).
// Symmetric, one fp32 scale per row: s = absmax / qmax (qmax 127 for int8,
// 448 for OCP e4m3; 1 for an all-zero row), code = round-to-nearest-even of
// the correctly rounded fp32 quotient h / s, saturated.  The quotient comes
// from one reciprocal per row and two fused multiply-adds per value: with
// r = RN(1/s) and q = RN(h*r), the remainder h - q*s is exact in an fma and
// RN(q + rem*r) is the correctly rounded quotient (Markstein's theorem on
// division by reciprocal refinement; it needs no overflow or underflow in
// the steps, which s >= 2^-60 and |h| <= qmax * s guarantee; rows with a
// smaller s take the plain division).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmoe {
namespace rq {

// Correctly rounded h / s given r = RN(1/s); `refine` is s >= 2^-60.
__device__ inline float quotient(float x, float s, float r, bool refine) {
  if (!refine) return x / s;
  const float q = x * r;
  return __builtin_fmaf(__builtin_fmaf(-q, s, x), r, q);
}

__device__ inline uint32_t to_e4m3x4(float a, float b, float c, float d) {
  // v_cvt_pk_fp8_f32: OCP e4m3 on gfx950, round to nearest even.  Inputs are
  // clamped to +-448 first so no value can round to NaN.
  a = fminf(fmaxf(a, -448.f), 448.f);
  b = fminf(fmaxf(b, -448.f), 448.f);
  c = fminf(fmaxf(c, -448.f), 448.f);
  d = fminf(fmaxf(d, -448.f), 448.f);
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
  return (uint32_t)v;
}

__device__ inline uint32_t to_i8x4(float a, float b, float c, float d) {
  const int qa = (int)fminf(fmaxf(rintf(a), -127.f), 127.f);
  const int qb = (int)fminf(fmaxf(rintf(b), -127.f), 127.f);
  const int qc = (int)fminf(fmaxf(rintf(c), -127.f), 127.f);
  const int qd = (int)fminf(fmaxf(rintf(d), -127.f), 127.f);
  return (uint32_t)(qa & 0xff) | ((uint32_t)(qb & 0xff) << 8) | ((uint32_t)(qc & 0xff) << 16) |
         ((uint32_t)(qd & 0xff) << 24);
}

// Codes of four consecutive h values of one row.
template <bool FP8>
__device__ inline uint32_t quant4(float a, float b, float c, float d, float s, float r,
                                  bool refine) {
  const float x0 = quotient(a, s, r, refine), x1 = quotient(b, s, r, refine);
  const float x2 = quotient(c, s, r, refine), x3 = quotient(d, s, r, refine);
  return FP8 ? to_e4m3x4(x0, x1, x2, x3) : to_i8x4(x0, x1, x2, x3);
}

// Row scale from the row's absmax.
template <bool FP8>
__device__ inline float row_scale(float absmax) {
  return absmax > 0.f ? absmax / (FP8 ? 448.0f : 127.0f) : 1.0f;
}

}  // namespace rq
}  // namespace qmoe
