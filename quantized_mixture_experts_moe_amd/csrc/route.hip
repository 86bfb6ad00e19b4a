// Top-k routing: k largest fp32 router logits per token (ties to the lower
// expert index), softmax renormalised over the k picked.  Top-k routing is
// named by the vLLM issue "Evaluate native IU4/IU8 WMMA for grouped-INT MoE
// prefill on gfx1151" (section Problem) and aiter PR 6090 (section Changes:
// topk 10); the tie rule and the renormalisation are this library's fixed
// reading.  The renormalised softmax over the picked experts equals the
// softmax of the picked logits because the full denominator cancels.
//
// One wave per token.  Each lane keeps EPL logits in registers (expert
// e = lane + 64*i) as 64-bit sortable keys: the high word orders the fp32
// values, the low word is ~e, so the largest key is the largest logit with
// the lowest index among equal ones.  k rounds of a wave-wide maximum pick
// the experts in slot order; the maximum runs on DPP row operations inside
// each 16-lane row and four lane reads across the rows (no LDS traffic).
// The weights use fp64 exp so that they match a correctly rounded fp32
// result.
#include "qmoe_internal.h"

namespace qmoe {
namespace {

typedef unsigned long long u64;

__device__ inline u64 make_key(float v, int e) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((u64)ord << 32) | (uint32_t)~(uint32_t)e;
}

__device__ inline float key_value(u64 k) {
  const uint32_t ord = (uint32_t)(k >> 32);
  const uint32_t b = (ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord;
  return __uint_as_float(b);
}

template <int CTRL>
__device__ inline u64 dpp_max(u64 x) {
  const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)x, CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(x >> 32), CTRL, 0xf, 0xf, false);
  const u64 y = ((u64)(uint32_t)hi << 32) | (uint32_t)lo;
  return y > x ? y : x;
}

// Maximum of x over the 64 lanes, returned in every lane.
__device__ inline u64 wave_max(u64 x) {
  x = dpp_max<0xB1>(x);   // quad_perm [1,0,3,2]
  x = dpp_max<0x4E>(x);   // quad_perm [2,3,0,1]
  x = dpp_max<0x141>(x);  // row_half_mirror: the two quads of each half-row
  x = dpp_max<0x140>(x);  // row_mirror: the two halves of each row
  u64 best = 0;
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, 16 * r);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), 16 * r);
    const u64 y = ((u64)hi << 32) | lo;
    best = y > best ? y : best;
  }
  return best;
}

template <int EPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T,
                                                    int E, int k, int32_t* __restrict__ ids,
                                                    float* __restrict__ wout) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave leaves together
  const float* row = logits + (size_t)t * E;
  u64 key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; i++) {
    const int e = lane + 64 * i;
    key[i] = e < E ? make_key(row[e], e) : 0ull;  // 0 sorts below every real key
  }
  float top0 = 0.f, my_v = 0.f;
  int my_e = 0;
  for (int j = 0; j < k; j++) {
    u64 mine = key[0];
#pragma unroll
    for (int i = 1; i < EPL; i++) mine = key[i] > mine ? key[i] : mine;
    const u64 best = wave_max(mine);
    const int bi = (int)~(uint32_t)best;
    const float bv = key_value(best);
    if ((bi & 63) == lane) {
#pragma unroll
      for (int i = 0; i < EPL; i++)
        if (i == (bi >> 6)) key[i] = 0ull;  // taken
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
