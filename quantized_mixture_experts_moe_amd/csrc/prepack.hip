// qmoe_prepack: canonical expert weights -> the streaming layout the grouped
// GEMM reads with QMOE_FLAG_PREPACKED.  Pure data movement (bytes; nibbles
// for W4A8).
//
// Canonical: row n of expert e is KB contiguous bytes (K along the row), its
// scales R contiguous bytes.  Streaming: for each group of 16 rows and each
// K step (S code bytes per row), one block of 16*S bytes in which lane
// L = 16*q + r of a wave finds, as its 16-byte piece i at i*1024 + L*16, the
// step bytes [64*i + 16*q, 64*i + 16*q + 16) of row r.  Each MFMA of a step
// then covers one contiguous K range (bytes [64*i, 64*i + 64)), which keeps
// the activation fragment reads free of LDS bank conflicts.  The two scale
// bytes of a lane sit at 128*ks + 2*L of the group's scale block: for A8W4
// the e8m0 bytes of 32-K blocks q and 4 + q of the step (one per MFMA), for
// W4A16 the fp16 scale of group q.
#include "qmoe_internal.h"

namespace qmoe {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// One thread per 16-byte output piece; grid-stride over all pieces.
// rows = E*N, KB = bytes per row, S = bytes per row per step.
__global__ void prepack_codes_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                     size_t rows, int KB, int S) {
  const size_t per_group = (size_t)KB;  // 16-byte pieces per 16-row group (16*KB bytes)
  const size_t total = rows / 16 * per_group;
  for (size_t oc = (size_t)blockIdx.x * blockDim.x + threadIdx.x; oc < total;
       oc += (size_t)gridDim.x * blockDim.x) {
    const size_t grp = oc / per_group;
    const int rem = (int)(oc - grp * per_group);  // piece inside the group
    const int ks = rem / S, rem2 = rem - ks * S;  // S pieces per step (16*S bytes)
    const int i = rem2 >> 6, L = rem2 & 63;
    const int q = L >> 4, r = L & 15;
    const size_t row = grp * 16 + r;
    const size_t sb = row * KB + (size_t)ks * S + i * 64 + q * 16;
    *reinterpret_cast<u32x4*>(dst + oc * 16) = *reinterpret_cast<const u32x4*>(src + sb);
  }
}

// One thread per 2-byte output entry.  R = scale bytes per row, nsteps =
// steps per row; fp16 (W4A16: one entry of 4 per step) or e8m0 (A8W4: the
// entries q and 4 + q of 8 per step).
__global__ void prepack_scales_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                      size_t rows, int R, bool e8m0, int nsteps) {
  const size_t per_group = (size_t)nsteps * 64;  // entries per 16-row group
  const size_t total = rows / 16 * per_group;
  for (size_t oc = (size_t)blockIdx.x * blockDim.x + threadIdx.x; oc < total;
       oc += (size_t)gridDim.x * blockDim.x) {
    const size_t grp = oc / per_group;
    const int rem = (int)(oc - grp * per_group);
    const int ks = rem >> 6, L = rem & 63;
    const int q = L >> 4, r = L & 15;
    const size_t row = grp * 16 + r;
    if (e8m0) {
      const uint8_t* p = src + row * R + (size_t)ks * 8;
      dst[oc * 2] = p[q];
      dst[oc * 2 + 1] = p[4 + q];
    } else {
      *reinterpret_cast<uint16_t*>(dst + oc * 2) =
          *reinterpret_cast<const uint16_t*>(src + row * R + (size_t)ks * 8 + q * 2);
    }
  }
}

// W4A8 codes, one thread per 4-byte output word: word j of lane L = 16q + r
// in step ks of a 16-row group holds, in byte b, K = 128 ks + 32 j + 8 q + b
// (low nibble) and K + 4 (high nibble) of row r.  Those eight K are the four
// canonical bytes at 64 ks + 16 j + 4 q of the row, nibble i of that word
// being K + i.
__global__ void prepack_w4a8_codes_kernel(const uint8_t* __restrict__ src,
                                          uint8_t* __restrict__ dst, size_t rows, int KB) {
  const size_t per_group = (size_t)KB * 4;  // 4-byte words per 16-row group
  const size_t total = rows / 16 * per_group;
  for (size_t ow = (size_t)blockIdx.x * blockDim.x + threadIdx.x; ow < total;
       ow += (size_t)gridDim.x * blockDim.x) {
    const size_t grp = ow / per_group;
    const int rem = (int)(ow - grp * per_group);
    const int ks = rem >> 8, L = (rem >> 2) & 63, j = rem & 3;
    const int q = L >> 4, r = L & 15;
    const size_t row = grp * 16 + r;
    const uint32_t w =
        *reinterpret_cast<const uint32_t*>(src + row * KB + (size_t)ks * 64 + j * 16 + q * 4);
    uint32_t o = 0;
#pragma unroll
    for (int b = 0; b < 4; b++) {
      const uint32_t lo = (w >> (4 * b)) & 0xFu, hi = (w >> (4 * (b + 4))) & 0xFu;
      o |= (lo | (hi << 4)) << (8 * b);
    }
    *reinterpret_cast<uint32_t*>(dst + ow * 4) = o;
  }
}

// W4A8 scales, one thread per 8-byte output entry (the four fp16 scales of
// a row's step): entry (group, ks, r) at group*16*R + ks*128 + r*8.
__global__ void prepack_w4a8_scales_kernel(const uint8_t* __restrict__ src,
                                           uint8_t* __restrict__ dst, size_t rows, int R,
                                           int nsteps) {
  const size_t per_group = (size_t)nsteps * 16;
  const size_t total = rows / 16 * per_group;
  for (size_t oe = (size_t)blockIdx.x * blockDim.x + threadIdx.x; oe < total;
       oe += (size_t)gridDim.x * blockDim.x) {
    const size_t grp = oe / per_group;
    const int rem = (int)(oe - grp * per_group);
    const int ks = rem >> 4, r = rem & 15;
    const size_t row = grp * 16 + r;
    *reinterpret_cast<unsigned long long*>(dst + oe * 8) =
        *reinterpret_cast<const unsigned long long*>(src + row * R + (size_t)ks * 8);
  }
}

int grid_for(size_t total) {
  const size_t want = (total + 255) / 256;
  const size_t cap = (size_t)device_cu_count() * 16;
  return (int)(want < cap ? (want > 0 ? want : 1) : cap);
}

}  // namespace

hipError_t launch_prepack(int scheme, int E, int N, int K, const void* codes, const void* scales,
                          void* codes_out, void* scales_out, hipStream_t s) {
  const size_t rows = (size_t)E * N;
  if (scheme == 3) {
    const int KB = K / 2, R = K / 32 * 2, nsteps = K / 128;
    const size_t words = rows / 16 * KB * 4;
    hipLaunchKernelGGL(prepack_w4a8_codes_kernel, dim3(grid_for(words)), dim3(256), 0, s,
                       reinterpret_cast<const uint8_t*>(codes),
                       reinterpret_cast<uint8_t*>(codes_out), rows, KB);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t entries = rows / 16 * nsteps * 16;
    hipLaunchKernelGGL(prepack_w4a8_scales_kernel, dim3(grid_for(entries)), dim3(256), 0, s,
                       reinterpret_cast<const uint8_t*>(scales),
                       reinterpret_cast<uint8_t*>(scales_out), rows, R, nsteps);
    return hipGetLastError();
  }
  const int KB = scheme == 1 ? K : K / 2;          // W8A8 int8, others 4-bit
  const int BK = scheme == 2 ? 256 : 128;          // K elements per step
  const int S = scheme == 1 ? BK : BK / 2;         // bytes per row per step
  const size_t pieces = rows / 16 * KB;
  hipLaunchKernelGGL(prepack_codes_kernel, dim3(grid_for(pieces)), dim3(256), 0, s,
                     reinterpret_cast<const uint8_t*>(codes), reinterpret_cast<uint8_t*>(codes_out),
                     rows, KB, S);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (scheme == 1) {
    if (scales_out == nullptr) return hipSuccess;
    return hipMemcpyAsync(scales_out, scales, rows * sizeof(float), hipMemcpyDeviceToDevice, s);
  }
  const int SB = scheme == 0 ? 2 : 1;
  const int R = K / 32 * SB;
  const int nsteps = K / BK;
  const size_t entries = rows / 16 * nsteps * 64;
  hipLaunchKernelGGL(prepack_scales_kernel, dim3(grid_for(entries)), dim3(256), 0, s,
                     reinterpret_cast<const uint8_t*>(scales),
                     reinterpret_cast<uint8_t*>(scales_out), rows, R, scheme == 2, nsteps);
  return hipGetLastError();
}

}  // namespace qmoe
