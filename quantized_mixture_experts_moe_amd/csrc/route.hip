// Top-k routing kernel: one wave per token (the routine and its reading are
// in route_common.h; vLLM issue "Evaluate native IU4/IU8 WMMA for
// grouped-INT MoE prefill on gfx1151", section Problem: top-k routing).
#include "qmoe_internal.h"
#include "route_common.h"

namespace qmoe {
namespace {

template <int EPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T,
                                                    int E, int k, int32_t* __restrict__ ids,
                                                    float* __restrict__ wout) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave leaves together
  int e;
  float w;
  rt::route_token<EPL>(logits + (size_t)t * E, E, k, &e, &w);
  if (lane < k) {
    ids[(size_t)t * k + lane] = e;
    wout[(size_t)t * k + lane] = w;
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
