// Top-k routing of one token by one wave (shared by the routing kernel and
// the fused small-batch routing + grouping kernel).  The k largest fp32
// router logits (ties to the lower expert index), softmax renormalised over
// the k picked: w_j = exp(L_j - L_0) / sum_i exp(L_i - L_0), in fp64, stored
// as fp32.  Top-k routing is named by the vLLM issue "Evaluate native
// IU4/IU8 WMMA for grouped-INT MoE prefill on gfx1151" (section Problem) and
// aiter PR 6090 (section Changes: topk 10); the tie rule and the
// renormalisation are this library's fixed reading.  The renormalised
// softmax over the picked experts equals the softmax of the picked logits
// because the full denominator cancels.
//
// Each lane keeps EPL logits in registers (expert e = lane + 64*i) as 32-bit
// order-preserving keys (0 marks a taken or missing expert; no finite logit
// maps to 0; -0 is keyed as +0, so that the two zeros tie as equal logits
// do).  Each of the k rounds takes the wave-wide maximum key, then the
// lowest expert index holding it (a wave-wide minimum): the largest logit,
// ties to the lower index.  Both reductions run on DPP row operations inside
// each 16-lane row and four lane reads across the rows (no LDS traffic).
// The weights use fp64 exp so that they match a correctly rounded fp32
// result.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmoe {
namespace rt {

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

// Routes the token whose logits start at `row` (E of them) with the calling
// wave; lane j < k returns slot j's expert in *e_out and weight in *w_out.
// Every lane of the wave must call it.
template <int EPL>
__device__ inline void route_token(const float* __restrict__ row, int E, int k, int* e_out,
                                   float* w_out) {
  const int lane = threadIdx.x & 63;
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
  *e_out = my_e;
  *w_out = (float)(ex / sum);
}

}  // namespace rt
}  // namespace qmoe
