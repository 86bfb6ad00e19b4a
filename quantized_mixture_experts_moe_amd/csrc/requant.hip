// Per-row requantization of the intermediate h for the activation-quantized
// schemes: w8a8 -> int8 (vLLM issue "Evaluate native IU4/IU8 WMMA for
// grouped-INT MoE prefill on gfx1151", section Constraint: integer matrix
// products need int8 activations), a8w4 -> fp8 e4m3 (aiter PR 6090, section
// Changes: fp8 act); the recipe is in quant_common.h.  This kernel serves the
// stage 2 that does not hold its rows in LDS (intermediate sizes above 1024);
// the resident stage 2 quantizes while it copies the rows.  The row absmax is
// the max of the per-column-tile maxima stage 1 wrote.  One wave per row;
// padding rows are skipped.
#include "qmoe_internal.h"
#include "quant_common.h"

namespace qmoe {
namespace {

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
  const float s = rq::row_scale<FP8>(a);
  if (lane == 0) hs[row] = s;
  const bool refine = s >= 0x1p-60f;  // the same for the whole wave
  const float r = 1.0f / s;
  for (int base = 0; base < n4; base += 64 * kVec) {
    if (base > 0) {
#pragma unroll
      for (int i = 0; i < kVec; i++)
        if (base + lane + 64 * i < n4) v[i] = src[base + lane + 64 * i];
    }
#pragma unroll
    for (int i = 0; i < kVec; i++) {
      const int idx = base + lane + 64 * i;
      if (idx < n4) dst[idx] = rq::quant4<FP8>(v[i].x, v[i].y, v[i].z, v[i].w, s, r, refine);
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
