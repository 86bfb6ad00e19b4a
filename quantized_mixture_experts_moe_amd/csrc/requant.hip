// Per-row requantization of the intermediate h for the activation-quantized
// schemes: w8a8 -> int8 (vLLM issue "Evaluate native IU4/IU8 WMMA for
// grouped-INT MoE prefill on gfx1151", section Constraint: integer matrix
// products need int8 activations), a8w4 -> fp8 e4m3 (aiter PR 6090, section
// Changes: fp8 act).  Symmetric, one fp32 scale per row:
//   s = absmax / qmax (qmax 127 or 448; 1 for an all-zero row),
//   w8a8: code = clamp(round_half_even(h / s), -127, 127)
//   a8w4: code = e4m3 round-to-nearest-even of h / s, saturated to +-448.
// The row absmax is the max of the per-column-tile maxima stage 1 wrote.
// One wave per row; padding rows are skipped.  h / s is the correctly
// rounded fp32 quotient, as a plain division gives, but from one reciprocal
// per row and two fused multiply-adds per value: with r = RN(1/s) and
// q = RN(h*r), the remainder h - q*s is exact in an fma and RN(q + rem*r)
// is the correctly rounded quotient (Markstein's theorem on division by
// reciprocal refinement; it needs no overflow or underflow in the steps,
// which s >= 2^-60 and |h| <= 448 s guarantee; rows with a smaller s use
// the plain division).
#include "qmoe_internal.h"

namespace qmoe {
namespace {

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

// A row is processed in passes of up to kVec*64 float4 (kVec*256 values);
// within a pass every load is issued before the row max is reduced, so a
// wave waits for memory about once per pass.
constexpr int kVec = 8;

template <bool FP8>
__global__ __launch_bounds__(256) void requant_kernel(const int32_t* __restrict__ sorted,
                                                      const int32_t* __restrict__ num_padded,
                                                      int P, int I, int ntiles_n,
                                                      const float* __restrict__ h32,
                                                      const float* __restrict__ pmax,
                                                      uint8_t* __restrict__ hq,
                                                      float* __restrict__ hs) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  // Both loads in one round trip: row < cap always (the grid is cap / 4
  // blocks and cap is a multiple of block_m), so sorted[row] is in bounds
  // even past num_padded.
  const int npad = *num_padded;
  const int pair = sorted[row];
  if (row >= npad || pair >= P) return;  // past the tiles, or a padding slot
  const float4* src = reinterpret_cast<const float4*>(h32 + (size_t)row * I);
  uint32_t* dst = reinterpret_cast<uint32_t*>(hq + (size_t)row * I);
  const int n4 = I / 4;
  float4 v[kVec];
#pragma unroll
  for (int i = 0; i < kVec; i++)
    if (lane + 64 * i < n4) v[i] = src[lane + 64 * i];
  float a = 0.f;
  for (int i = lane; i < ntiles_n; i += 64) a = fmaxf(a, pmax[(size_t)row * ntiles_n + i]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
  const float s = a > 0.f ? a / (FP8 ? 448.0f : 127.0f) : 1.0f;
  if (lane == 0) hs[row] = s;
  const bool refine = s >= 0x1p-60f;  // the same for the whole wave
  const float r = 1.0f / s;
  auto quot = [&](float x) __attribute__((always_inline)) {
    if (!refine) return x / s;
    const float q = x * r;
    return __builtin_fmaf(__builtin_fmaf(-q, s, x), r, q);
  };
  for (int base = 0; base < n4; base += 64 * kVec) {
    if (base > 0) {
#pragma unroll
      for (int i = 0; i < kVec; i++)
        if (base + lane + 64 * i < n4) v[i] = src[base + lane + 64 * i];
    }
#pragma unroll
    for (int i = 0; i < kVec; i++) {
      const int idx = base + lane + 64 * i;
      if (idx < n4) {
        const float x0 = quot(v[i].x), x1 = quot(v[i].y), x2 = quot(v[i].z), x3 = quot(v[i].w);
        dst[idx] = FP8 ? to_e4m3x4(x0, x1, x2, x3) : to_i8x4(x0, x1, x2, x3);
      }
    }
  }
}

}  // namespace

hipError_t launch_requant(int scheme, const int32_t* sorted, const int32_t* num_padded, int P,
                          int I, int ntiles_n, int cap, const float* h32, const float* pmax,
                          uint8_t* hq, float* hs, hipStream_t s) {
  if (cap % 4 != 0) return hipErrorInvalidValue;  // every row of the grid must be below cap
  const dim3 grid(cap / 4), block(256);
  if (scheme == 2)
    hipLaunchKernelGGL(requant_kernel<true>, grid, block, 0, s, sorted, num_padded, P, I,
                       ntiles_n, h32, pmax, hq, hs);
  else
    hipLaunchKernelGGL(requant_kernel<false>, grid, block, 0, s, sorted, num_padded, P, I,
                       ntiles_n, h32, pmax, hq, hs);
  return hipGetLastError();
}

}  // namespace qmoe
