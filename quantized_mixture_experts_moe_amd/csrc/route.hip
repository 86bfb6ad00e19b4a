// Top-k routing: k largest fp32 router logits per token (ties to the lower
// expert index), softmax renormalised over the k picked.  Top-k routing is
// named by the vLLM issue "Evaluate native IU4/IU8 WMMA for grouped-INT MoE
// prefill on gfx1151" (section Problem) and aiter PR 6090 (section Changes:
// topk 10); the tie rule and the renormalisation are this library's fixed
// reading.  The renormalised softmax over the picked experts equals the
// softmax of the picked logits because the full denominator cancels.
//
// One wave per token.  Each lane keeps EPL logits in registers (expert
// e = lane + 64*i); k rounds of a wave-wide arg-max with (value desc, index
// asc) ordering pick the experts in slot order.  The weights use fp64 exp
// so that they match a correctly rounded fp32 result.
#include "qmoe_internal.h"

namespace qmoe {
namespace {

__device__ inline bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

template <int EPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T,
                                                    int E, int k, int32_t* __restrict__ ids,
                                                    float* __restrict__ wout) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave leaves together
  const float* row = logits + (size_t)t * E;
  float v[EPL];
#pragma unroll
  for (int i = 0; i < EPL; i++) {
    const int e = lane + 64 * i;
    v[i] = e < E ? row[e] : -__builtin_huge_valf();
  }
  uint64_t taken = 0;
  float top0 = 0.f, my_v = 0.f;
  int my_e = 0;
  for (int j = 0; j < k; j++) {
    float bv = -__builtin_huge_valf();
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < EPL; i++) {
      const int e = lane + 64 * i;
      if (e < E && !((taken >> i) & 1) && better(v[i], e, bv, bi)) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1ull << (bi >> 6);
    if (j == 0) top0 = bv;
    if (lane == j) {
      my_v = bv;
      my_e = bi;
    }
  }
  // Slot j lives in lane j.  The denominator is summed in slot order.
  const double ex = lane < k ? exp((double)my_v - (double)top0) : 0.0;
  double sum = 0.0;
  for (int j = 0; j < k; j++) sum += __shfl(ex, j, 64);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_e;
    wout[(size_t)t * k + lane] = (float)(ex / sum);
  }
}

}  // namespace

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                        hipStream_t s) {
  const dim3 grid((T + 3) / 4), block(256);
#define QMOE_ROUTE_CASE(EPL)                                                         \
  if (E <= 64 * EPL) {                                                               \
    hipLaunchKernelGGL(route_kernel<EPL>, grid, block, 0, s, logits, T, E, k, ids, w); \
    return hipGetLastError();                                                        \
  }
  QMOE_ROUTE_CASE(1)
  QMOE_ROUTE_CASE(2)
  QMOE_ROUTE_CASE(4)
  QMOE_ROUTE_CASE(8)
  QMOE_ROUTE_CASE(16)
#undef QMOE_ROUTE_CASE
  return hipErrorInvalidValue;
}

}  // namespace qmoe
