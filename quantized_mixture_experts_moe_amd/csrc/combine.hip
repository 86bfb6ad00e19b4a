// Weighted combine in a fixed order with no atomics (hip-ep PR "perf(qmoe):
// group prefill expert matmuls", description: deterministic scatter order):
//   out[t, :] = sum_{j=0}^{k-1} w[t, j] * y_pairs[t*k + j, :]
// accumulated in fp32 as acc = acc + (w * y), j ascending, no fused
// multiply-add, so every element's result is bitwise reproducible.
// Each thread produces 8 consecutive columns of one token; the k expert rows
// of a token are adjacent in y_pairs (row = pair id), so a block streams
// them with 16- or 32-byte loads.
#include "qmoe_internal.h"

namespace qmoe {
namespace {

__device__ inline void load8(const void* y, bool f32, size_t idx, float v[8]) {
  if (f32) {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(y) + idx);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 q = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(y) + idx);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
}

template <bool F32>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y,
                                                      const float* __restrict__ w, int T, int k,
                                                      int H, uint16_t* __restrict__ out_bf16,
                                                      float* __restrict__ out_f32) {
  const int groups = H / 8;
  const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (size_t)T * groups) return;
  const int t = (int)(gid / groups);
  const int c = (int)(gid - (size_t)t * groups) * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; j++) {
    const float wj = w[(size_t)t * k + j];
    float v[8];
    load8(y, F32, ((size_t)t * k + j) * H + c, v);
#pragma unroll
    for (int i = 0; i < 8; i++) acc[i] = acc[i] + wj * v[i];  // built with -ffp-contract=off
  }
  const size_t o = (size_t)t * H + c;
  if (out_f32 != nullptr) {
    float4* p = reinterpret_cast<float4*>(out_f32 + o);
    p[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    p[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
  if (out_bf16 != nullptr) {
    uint32_t pk[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const __bf16 lo = (__bf16)acc[2 * i], hi = (__bf16)acc[2 * i + 1];
      pk[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
              ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    *reinterpret_cast<uint4*>(out_bf16 + o) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  }
}

}  // namespace

hipError_t launch_combine(const void* y, int y_f32, const float* w, int T, int k, int H,
                          uint16_t* out_bf16, float* out_f32, hipStream_t s) {
  const size_t n = (size_t)T * (H / 8);
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
  if (y_f32)
    hipLaunchKernelGGL(combine_kernel<true>, grid, block, 0, s, y, w, T, k, H, out_bf16, out_f32);
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, block, 0, s, y, w, T, k, H, out_bf16, out_f32);
  return hipGetLastError();
}

}  // namespace qmoe
