// moe_align: group the P = T*k (token, slot) pairs by expert, stable in pair
// id, each expert padded to a multiple of block_m with the sentinel P.
// This is what lets one launch per projection cover every expert (hip-ep PR
// "perf(qmoe): group prefill expert matmuls", description: expert
// projections batched into single launches, deterministic scatter order).
//
// A token's k experts are distinct, so the rank of pair (t, j) inside expert
// e is the number of earlier tokens routed to e.  Three small kernels:
//  1. count: one block per 256-token chunk; each wave builds in LDS a 64-bit
//     mask per expert of its 64 tokens routed to that expert, and the block
//     writes the chunk's count per expert, counts[e][chunk].
//  2. scan: one block.  A wave scans an expert's chunk counts into chunk
//     bases (exclusive prefix), the expert totals are padded to block_m and
//     scanned into expert offsets; the tile->expert map and the sentinels of
//     the padding are written.
//  3. scatter: the count blocks again; a pair's slot is the expert offset +
//     the chunk base + the earlier waves' counts + popcount(mask & lanes
//     below).
#include "qmoe_internal.h"

namespace qmoe {
namespace {

constexpr int kChunk = 256;        // tokens per count/scatter block
constexpr int kMaxExperts = 1024;  // LDS bound of the mask arrays and the scan block

// Builds the per-wave expert masks of this block's 256 tokens; returns, in
// every thread, the block's flag bits: 1 = an expert id outside [0, E),
// 2 = an expert repeated within one token's k ids.
__device__ inline int build_masks(const int32_t* __restrict__ ids, int T, int k, int E,
                                  unsigned long long* mask) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int i = tid; i < 4 * E; i += kChunk) mask[i] = 0ull;
  __syncthreads();
  const int t = blockIdx.x * kChunk + tid;
  int bad = 0;
  if (t < T) {
    for (int j = 0; j < k; j++) {
      const int e = ids[(size_t)t * k + j];
      if (e >= 0 && e < E) {
        const unsigned long long old = atomicOr(&mask[wave * E + e], 1ull << lane);
        if (old & (1ull << lane)) bad |= 2;
      } else {
        bad |= 1;
      }
    }
  }
  __syncthreads();
  // Block-wide OR of the two flag bits.
  const int b1 = __syncthreads_or(bad & 1);
  const int b2 = __syncthreads_or(bad & 2);
  return (b1 ? 1 : 0) | (b2 ? 2 : 0);
}

__global__ __launch_bounds__(kChunk) void align_count_kernel(const int32_t* __restrict__ ids,
                                                              int T, int k, int E, int nchunks,
                                                              int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ chunk_flags) {
  extern __shared__ unsigned long long mask[];  // [4][E]
  const int bad = build_masks(ids, T, k, E, mask);
  if (threadIdx.x == 0) chunk_flags[blockIdx.x] = bad;
  for (int e = threadIdx.x; e < E; e += kChunk) {
    const int c = __popcll(mask[e]) + __popcll(mask[E + e]) + __popcll(mask[2 * E + e]) +
                  __popcll(mask[3 * E + e]);
    counts[(size_t)e * nchunks + blockIdx.x] = c;
  }
}

__global__ __launch_bounds__(1024) void align_scan_kernel(int nchunks, int E, int block_m, int P,
                                                          int cap, int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ sorted,
                                                          int32_t* __restrict__ tile_expert,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ num_padded,
                                                          const int32_t* __restrict__ chunk_flags,
                                                          int32_t* __restrict__ flags) {
  __shared__ int s_total[kMaxExperts];
  __shared__ int s_part[1024];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  constexpr int kBatch = 8;  // experts whose loads a wave keeps in flight together
  for (int eb = wave * kBatch; eb < E; eb += 16 * kBatch) {
    int carry[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; i++) carry[i] = 0;
    for (int cg = 0; cg < nchunks; cg += 64) {
      const int c = cg + lane;
      int v[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; i++) {
        const int e = eb + i;
        v[i] = (e < E && c < nchunks) ? counts[(size_t)e * nchunks + c] : 0;
      }
#pragma unroll
      for (int i = 0; i < kBatch; i++) {
        int x = v[i];
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int y = __shfl_up(x, off, 64);
          if (lane >= off) x += y;
        }
        const int e = eb + i;
        if (e < E && c < nchunks) counts[(size_t)e * nchunks + c] = carry[i] + x - v[i];
        carry[i] += __shfl(x, 63, 64);
      }
    }
#pragma unroll
    for (int i = 0; i < kBatch; i++)
      if (lane == 0 && eb + i < E) s_total[eb + i] = carry[i];
  }
  __syncthreads();
  // Each thread owns a contiguous run of experts [e0, e1).
  const int per = (E + 1023) / 1024;
  const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
  int run_pad = 0;
  for (int e = e0; e < e1; e++) run_pad += (s_total[e] + block_m - 1) / block_m * block_m;
  s_part[tid] = run_pad;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive scan of the run totals
    const int v = tid >= off ? s_part[tid - off] : 0;
    __syncthreads();
    s_part[tid] += v;
    __syncthreads();
  }
  const int npad = s_part[1023];
  int base = s_part[tid] - run_pad;
  for (int e = e0; e < e1; e++) {
    const int total = s_total[e];
    const int padded = (total + block_m - 1) / block_m * block_m;
    offsets[e] = base;
    for (int i = base / block_m; i < (base + padded) / block_m; i++) tile_expert[i] = e;
    for (int i = base + total; i < base + padded; i++) sorted[i] = P;
    base += padded;
  }
  int bad = 0;
  for (int c = tid; c < nchunks; c += 1024) bad |= chunk_flags[c];
  const int b1 = __syncthreads_or(bad & 1);
  const int b2 = __syncthreads_or(bad & 2);
  if (tid == 0) {
    offsets[E] = npad;
    *num_padded = npad;
    *flags = (b1 ? 1 : 0) | (b2 ? 2 : 0);
  }
  for (int i = npad + tid; i < cap; i += 1024) sorted[i] = P;
  for (int i = npad / block_m + tid; i < cap / block_m; i += 1024) tile_expert[i] = -1;
}

__global__ __launch_bounds__(kChunk) void align_scatter_kernel(
    const int32_t* __restrict__ ids, int T, int k, int E, int nchunks,
    const int32_t* __restrict__ chunk_base, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted) {
  extern __shared__ unsigned long long mask[];  // [4][E]
  build_masks(ids, T, k, E, mask);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int t = blockIdx.x * kChunk + tid;
  if (t >= T) return;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int j = 0; j < k; j++) {
    const int e = ids[(size_t)t * k + j];
    if (e < 0 || e >= E) continue;
    int rank = __popcll(mask[wave * E + e] & below);
    for (int w = 0; w < wave; w++) rank += __popcll(mask[w * E + e]);
    sorted[offsets[e] + chunk_base[(size_t)e * nchunks + blockIdx.x] + rank] = t * k + j;
  }
}

}  // namespace

hipError_t launch_align(const int32_t* ids, int T, int k, int E, int block_m, int32_t* sorted,
                        int32_t* tile_expert, int32_t* offsets, int32_t* num_padded,
                        int32_t* chunk_counts, int32_t* chunk_flags, int32_t* flags, int cap,
                        hipStream_t s) {
  if (E > kMaxExperts) return hipErrorInvalidValue;
  const int nchunks = (T + kChunk - 1) / kChunk;
  const size_t lds = (size_t)4 * E * sizeof(unsigned long long);
  hipError_t err;
  if (nchunks > 0) {
    hipLaunchKernelGGL(align_count_kernel, dim3(nchunks), dim3(kChunk), lds, s, ids, T, k, E,
                       nchunks, chunk_counts, chunk_flags);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(align_scan_kernel, dim3(1), dim3(1024), 0, s, nchunks, E, block_m, T * k,
                     cap, chunk_counts, sorted, tile_expert, offsets, num_padded, chunk_flags,
                     flags);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (nchunks == 0) return hipSuccess;
  hipLaunchKernelGGL(align_scatter_kernel, dim3(nchunks), dim3(kChunk), lds, s, ids, T, k, E,
                     nchunks, chunk_counts, offsets, sorted);
  return hipGetLastError();
}

size_t align_chunk_count(int T) { return (size_t)(T + kChunk - 1) / kChunk; }

}  // namespace qmoe
