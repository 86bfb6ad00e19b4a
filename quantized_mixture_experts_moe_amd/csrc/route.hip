// Top-k routing: k largest fp32 router logits per token (ties to the lower
// expert index), softmax renormalised over the k picked.  Top-k routing is
// named by the vLLM issue "Evaluate native IU4/IU8 WMMA for grouped-INT MoE
// prefill on gfx1151" (section Problem) and aiter PR 6090 (section Changes:
// topk 10); the tie rule and the renormalisation are this library's fixed
// reading.  The renormalised softmax over the picked experts equals the
// softmax of the picked logits because the full denominator cancels.
//
// One wave per token.  Each lane keeps EPL logits in registers (expert
// e = lane + 64*i) as 32-bit order-preserving keys (0 marks a taken or
// missing expert; no finite logit maps to 0; -0 is keyed as +0, so that
// the two zeros tie as equal logits do).  Each of the k rounds takes
// the wave-wide maximum key, then the lowest expert index holding it (a
// wave-wide minimum): the largest logit, ties to the lower index.  Both
// reductions run on DPP row operations inside each 16-lane row and four
// lane reads across the rows (no LDS traffic).  The weights use fp64 exp
// so that they match a correctly rounded fp32 result.
#include "qmoe_internal.h"

namespace qmoe {
namespace {

__device__ inline uint32_t order_key(float v) {
  const uint32_t b = __float_as_uint(v + 0.0f);  // -0 + +0 = +0 (round to nearest)
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ inline float key_value(uint32_t ord) {
  const uint32_t b = (ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord;
  return __uint_as_float(b);
}

// x combined with the lane that DPP control CTRL names, by MAX or min.
template <int CTRL, bool MAX>
__device__ inline uint32_t dpp_op(uint32_t x) {
  const uint32_t y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xf, 0xf, false);
  return MAX ? (y > x ? y : x) : (y < x ? y : x);
}

// Maximum (MAX) or minimum of x over the 64 lanes, in every lane.
template <bool MAX>
__device__ inline uint32_t wave_reduce(uint32_t x) {
  x = dpp_op<0xB1, MAX>(x);   // quad_perm [1,0,3,2]
  x = dpp_op<0x4E, MAX>(x);   // quad_perm [2,3,0,1]
  x = dpp_op<0x141, MAX>(x);  // row_half_mirror: the two quads of each half-row
  x = dpp_op<0x140, MAX>(x);  // row_mirror: the two halves of each row
  uint32_t r = (uint32_t)__builtin_amdgcn_readlane((int)x, 0);
#pragma unroll
  for (int row = 1; row < 4; row++) {
    const uint32_t y = (uint32_t)__builtin_amdgcn_readlane((int)x, 16 * row);
    r = MAX ? (y > r ? y : r) : (y < r ? y : r);
  }
  return r;
}

template <int EPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T,
                                                    int E, int k, int32_t* __restrict__ ids,
                                                    float* __restrict__ wout) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave leaves together
  const float* row = logits + (size_t)t * E;
  uint32_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; i++) {
    const int e = lane + 64 * i;
    key[i] = e < E ? order_key(row[e]) : 0u;
  }
  float top0 = 0.f, my_v = 0.f;
  int my_e = 0;
  for (int j = 0; j < k; j++) {
    uint32_t mine = key[0];
#pragma unroll
    for (int i = 1; i < EPL; i++) mine = key[i] > mine ? key[i] : mine;
    const uint32_t best = wave_reduce<true>(mine);
    // This lane's lowest expert holding the maximum (0xffffffff if none),
    // then the lowest over the wave.
    uint32_t cand = 0xffffffffu;
#pragma unroll
    for (int i = EPL - 1; i >= 0; i--)
      if (key[i] == best) cand = (uint32_t)(lane + 64 * i);
    const int bi = (int)wave_reduce<false>(cand);
    const float bv = key_value(best);
    if ((bi & 63) == lane) {
#pragma unroll
      for (int i = 0; i < EPL; i++)
        if (i == (bi >> 6)) key[i] = 0u;  // taken
    }
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
