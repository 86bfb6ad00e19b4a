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

typedef unsigned v4u __attribute__((ext_vector_type(4)));

// Raw 16 or 32 bytes of 8 consecutive y values, loaded once (streaming).
template <bool F32>
struct Raw8 {
  v4u q[F32 ? 2 : 1];
};

template <bool F32>
__device__ inline Raw8<F32> load8(const void* y, size_t idx) {
  Raw8<F32> r;
  if constexpr (F32) {
    const v4u* p = reinterpret_cast<const v4u*>(reinterpret_cast<const float*>(y) + idx);
    r.q[0] = __builtin_nontemporal_load(p);
    r.q[1] = __builtin_nontemporal_load(p + 1);
  } else {
    r.q[0] = __builtin_nontemporal_load(
        reinterpret_cast<const v4u*>(reinterpret_cast<const uint16_t*>(y) + idx));
  }
  return r;
}

template <bool F32>
__device__ inline void unpack8(const Raw8<F32>& r, float v[8]) {
  if constexpr (F32) {
    const uint32_t w[8] = {r.q[0].x, r.q[0].y, r.q[0].z, r.q[0].w,
                           r.q[1].x, r.q[1].y, r.q[1].z, r.q[1].w};
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = __uint_as_float(w[i]);
  } else {
    const uint32_t w[4] = {r.q[0].x, r.q[0].y, r.q[0].z, r.q[0].w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
}

// The k rows of a token are read in groups of KU, all loads of a group
// issued before the first of them is used.
template <bool F32>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y,
                                                      const float* __restrict__ w, int T, int k,
                                                      int H, uint16_t* __restrict__ out_bf16,
                                                      float* __restrict__ out_f32) {
  constexpr int KU = F32 ? 8 : 16;
  const int groups = H / 8;
  const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (size_t)T * groups) return;
  const int t = (int)(gid / groups);
  const int c = (int)(gid - (size_t)t * groups) * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < k; j0 += KU) {
    Raw8<F32> raw[KU];
    float wj[KU];
#pragma unroll
    for (int u = 0; u < KU; u++) {
      if (j0 + u < k) {
        raw[u] = load8<F32>(y, ((size_t)t * k + j0 + u) * H + c);
        wj[u] = w[(size_t)t * k + j0 + u];
      }
    }
#pragma unroll
    for (int u = 0; u < KU; u++) {
      if (j0 + u < k) {
        float v[8];
        unpack8<F32>(raw[u], v);
#pragma unroll
        for (int i = 0; i < 8; i++) acc[i] = acc[i] + wj[u] * v[i];  // built with -ffp-contract=off
      }
    }
  }
  const size_t o = (size_t)t * H + c;
  if (out_f32 != nullptr) {
    v4u* p = reinterpret_cast<v4u*>(out_f32 + o);
    __builtin_nontemporal_store(v4u{__float_as_uint(acc[0]), __float_as_uint(acc[1]),
                                    __float_as_uint(acc[2]), __float_as_uint(acc[3])},
                                p);
    __builtin_nontemporal_store(v4u{__float_as_uint(acc[4]), __float_as_uint(acc[5]),
                                    __float_as_uint(acc[6]), __float_as_uint(acc[7])},
                                p + 1);
  }
  if (out_bf16 != nullptr) {
    uint32_t pk[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const __bf16 lo = (__bf16)acc[2 * i], hi = (__bf16)acc[2 * i + 1];
      pk[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
              ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    __builtin_nontemporal_store(v4u{pk[0], pk[1], pk[2], pk[3]},
                                reinterpret_cast<v4u*>(out_bf16 + o));
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
