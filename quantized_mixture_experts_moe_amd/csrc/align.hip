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
//  2. scan: one block.  Each expert's chunk counts become chunk bases
//     (exclusive prefix, staged through LDS), the expert totals are padded to
//     block_m and scanned into expert offsets.
//  3. scatter: the count blocks again; a pair's slot is the expert offset +
//     the chunk base + the earlier waves' counts + popcount(mask & lanes
//     below).  The same launch writes the padding sentinels, the
//     tile->expert map and the tail, spread over at least 32 blocks.
// Up to 512 tokens all three steps run in one block of one launch
// (align_small_kernel): short prefills pay one launch, not three.  Up to
// 64 chunks (16384 tokens) the scan runs inside the scatter launch
// (align_place_kernel): every block reads the whole count matrix and scans
// it itself, so two launches remain.
#include "qmoe_internal.h"
#include "route_common.h"

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

// Chunk counts staged in LDS per scan pass: the experts of a pass are those
// whose nchunks counts fit (row pitch nchunks + 1 keeps the per-expert
// walks free of bank conflicts).
constexpr int kScanLdsInts = 16384;

__global__ __launch_bounds__(1024) void align_scan_kernel(int nchunks, int E, int block_m,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ totals,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ num_padded,
                                                          const int32_t* __restrict__ chunk_flags,
                                                          int32_t* __restrict__ flags) {
  __shared__ int s_cnt[kScanLdsInts];
  __shared__ int s_total[kMaxExperts];
  __shared__ int s_part[1024];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // 1. counts[e][c] -> exclusive prefix over c (the chunk bases), in place,
  //    and the expert totals.  Passes of experts whose counts fit in LDS:
  //    one coalesced load, one thread per expert walks its row, one
  //    coalesced store.
  const int pitch = nchunks + 1;
  const int per_pass = max(1, min(E, kScanLdsInts / pitch));
  for (int e0 = 0; e0 < E; e0 += per_pass) {
    const int ne = min(per_pass, E - e0);
    const int n = ne * nchunks;
    const int32_t* src = counts + (size_t)e0 * nchunks;
    if (pitch * ne <= kScanLdsInts) {
      for (int i = tid; i < n; i += 1024) s_cnt[(i / nchunks) * pitch + i % nchunks] = src[i];
      __syncthreads();
      for (int e = tid; e < ne; e += 1024) {
        int run = 0;
        int* row = s_cnt + e * pitch;
        for (int c = 0; c < nchunks; c++) {
          const int v = row[c];
          row[c] = run;
          run += v;
        }
        s_total[e0 + e] = run;
      }
      __syncthreads();
      int32_t* dst = counts + (size_t)e0 * nchunks;
      for (int i = tid; i < n; i += 1024) dst[i] = s_cnt[(i / nchunks) * pitch + i % nchunks];
      __syncthreads();
    } else {
      // One expert's row exceeds LDS (more than kScanLdsInts chunks): a
      // wave scans each row in pieces of 64 chunks.
      for (int e = e0 + wave; e < e0 + ne; e += 16) {
        int carry = 0;
        int32_t* row = counts + (size_t)e * nchunks;
        for (int cg = 0; cg < nchunks; cg += 64) {
          const int c = cg + lane;
          const int v = c < nchunks ? row[c] : 0;
          int x = v;
#pragma unroll
          for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
          }
          if (c < nchunks) row[c] = carry + x - v;
          carry += __shfl(x, 63, 64);
        }
        if (lane == 0) s_total[e] = carry;
      }
      __syncthreads();
    }
  }
  // 2. Expert offsets: exclusive scan of the block_m-padded totals.  Each
  //    thread owns a contiguous run of experts.
  const int per = (E + 1023) / 1024;
  const int r0 = min(E, tid * per), r1 = min(E, r0 + per);
  int run_pad = 0;
  for (int e = r0; e < r1; e++) run_pad += (s_total[e] + block_m - 1) / block_m * block_m;
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
  for (int e = r0; e < r1; e++) {
    offsets[e] = base;
    totals[e] = s_total[e];
    base += (s_total[e] + block_m - 1) / block_m * block_m;
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
}

// Blocks below nchunks place their chunk's pairs; every block then takes a
// share of the padding: the sentinels after each expert's pairs and its
// tile->expert entries (one wave per expert, consecutive lanes on
// consecutive slots), and the tail from num_padded to cap.
__global__ __launch_bounds__(kChunk) void align_scatter_kernel(
    const int32_t* __restrict__ ids, int T, int k, int E, int nchunks, int block_m, int cap,
    const int32_t* __restrict__ chunk_base, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ totals, int32_t* __restrict__ sorted,
    int32_t* __restrict__ tile_expert) {
  extern __shared__ unsigned long long mask[];  // [4][E]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int P = T * k;
  if ((int)blockIdx.x < nchunks) {
    build_masks(ids, T, k, E, mask);
    const int t = blockIdx.x * kChunk + tid;
    if (t < T) {
      const unsigned long long below = (1ull << lane) - 1ull;
      for (int j = 0; j < k; j++) {
        const int e = ids[(size_t)t * k + j];
        if (e < 0 || e >= E) continue;
        int rank = __popcll(mask[wave * E + e] & below);
        for (int w = 0; w < wave; w++) rank += __popcll(mask[w * E + e]);
        sorted[offsets[e] + chunk_base[(size_t)e * nchunks + blockIdx.x] + rank] = t * k + j;
      }
    }
  }
  const int nwaves = gridDim.x * (kChunk / 64);
  for (int e = blockIdx.x * (kChunk / 64) + wave; e < E; e += nwaves) {
    const int off = offsets[e], total = totals[e];
    const int padded = (total + block_m - 1) / block_m * block_m;
    for (int i = off / block_m + lane; i < (off + padded) / block_m; i += 64) tile_expert[i] = e;
    for (int i = off + total + lane; i < off + padded; i += 64) sorted[i] = P;
  }
  const int npad = offsets[E];
  const int stride = gridDim.x * kChunk;
  for (int i = npad + blockIdx.x * kChunk + tid; i < cap; i += stride) sorted[i] = P;
  for (int i = npad / block_m + blockIdx.x * kChunk + tid; i < cap / block_m; i += stride)
    tile_expert[i] = -1;
}

// The whole of moe_align for up to kSmallT tokens in one block of 16 waves
// (64 tokens each; the launcher sends it at most 512): masks, expert totals (one expert per thread), the padded
// offsets (block scan), the scatter, the padding sentinels, the
// tile->expert map and the tail.  block_m is a power of two.
constexpr int kSmallT = 1024;
constexpr int kSmallWaves = kSmallT / 64;

// Exclusive prefix sum of v over the block (any size up to 1024 threads);
// s_wave holds one int per wave.
__device__ inline int block_excl_scan(int v, int* s_wave) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; w++) before += s_wave[w];
  return before + x - v;
}

// Body of the single-block align; getid(t, j) returns token t's j-th id.
template <typename GetId>
__device__ inline void align_small_body(GetId getid, int T, int k, int E, int bm_shift, int cap,
                                        int32_t* __restrict__ sorted,
                                        int32_t* __restrict__ tile_expert,
                                        int32_t* __restrict__ offsets,
                                        int32_t* __restrict__ num_padded,
                                        int32_t* __restrict__ flags) {
  extern __shared__ unsigned long long mask[];  // [kSmallWaves][E]
  __shared__ int s_tot[kMaxExperts];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_wave[kSmallWaves];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int P = T * k;
  const int bm = 1 << bm_shift;
  const bool mine = tid < T;
  // This thread's token ids (up to kRegK of them kept in registers), all
  // loads issued before the mask is cleared so that their round trips
  // overlap each other and the clearing.
  constexpr int kRegK = 16;
  int te[kRegK];
#pragma unroll
  for (int j = 0; j < kRegK; j++) te[j] = mine && j < k ? getid(tid, j) : -1;
  for (int i = tid; i < kSmallWaves * E; i += kSmallT) mask[i] = 0ull;
  __syncthreads();
  int bad = 0;
  auto set_bit = [&](int e) __attribute__((always_inline)) {
    if (e >= 0 && e < E) {
      const unsigned long long old = atomicOr(&mask[wave * E + e], 1ull << lane);
      if (old & (1ull << lane)) bad |= 2;
    } else {
      bad |= 1;
    }
  };
#pragma unroll
  for (int j = 0; j < kRegK; j++)
    if (mine && j < k) set_bit(te[j]);
  for (int j = kRegK; j < k; j++)
    if (mine) set_bit(getid(tid, j));
  const int b1 = __syncthreads_or(bad & 1);
  const int b2 = __syncthreads_or(bad & 2);
  // Totals, one expert per thread (E <= 1024), and their padded prefix.
  int tot = 0;
  if (tid < E) {
#pragma unroll 4
    for (int w = 0; w < kSmallWaves; w++) tot += __popcll(mask[w * E + tid]);
  }
  const int pe = ((tot + bm - 1) >> bm_shift) << bm_shift;
  const int off = block_excl_scan(tid < E ? pe : 0, s_wave);
  if (tid < E) {
    s_tot[tid] = tot;
    s_off[tid] = off;
    offsets[tid] = off;
  }
  if (tid == E - 1) {
    s_off[E] = off + pe;
    offsets[E] = off + pe;
    *num_padded = off + pe;
    *flags = (b1 ? 1 : 0) | (b2 ? 2 : 0);
  }
  __syncthreads();
  // Scatter: rank inside the expert = pairs of earlier tokens.
  const unsigned long long below = (1ull << lane) - 1ull;
  auto place = [&](int e, int j) __attribute__((always_inline)) {
    if (e < 0 || e >= E) return;
    int rank = __popcll(mask[wave * E + e] & below);
    for (int w = 0; w < wave; w++) rank += __popcll(mask[w * E + e]);
    sorted[s_off[e] + rank] = tid * k + j;
  };
#pragma unroll
  for (int j = 0; j < kRegK; j++)
    if (mine && j < k) place(te[j], j);
  for (int j = kRegK; j < k; j++)
    if (mine) place(getid(tid, j), j);
  // Sentinels and tile->expert entries: a group of block_m / 4 lanes (4 to
  // 32) per expert, so that an expert's at most block_m - 1 sentinels take
  // at most four stores per lane and a wave serves 64 / group experts at a
  // time.
  {
    const int gs_shift = bm_shift - 2;  // block_m is 16..128
    const int gs = 1 << gs_shift, per_wave = 64 >> gs_shift;
    const int sub = lane >> gs_shift, sl = lane & (gs - 1);
    for (int e = wave * per_wave + sub; e < E; e += kSmallWaves * per_wave) {
      const int o = s_off[e], t = s_tot[e], end = s_off[e + 1];
      for (int i = (o >> bm_shift) + sl; i < (end >> bm_shift); i += gs) tile_expert[i] = e;
      for (int i = o + t + sl; i < end; i += gs) sorted[i] = P;
    }
  }
  const int npad = s_off[E];
  for (int i = npad + tid; i < cap; i += kSmallT) sorted[i] = P;
  for (int i = (npad >> bm_shift) + tid; i < (cap >> bm_shift); i += kSmallT) tile_expert[i] = -1;
}

__global__ __launch_bounds__(kSmallT) void align_small_kernel(
    const int32_t* __restrict__ ids, int T, int k, int E, int bm_shift, int cap,
    int32_t* __restrict__ sorted, int32_t* __restrict__ tile_expert,
    int32_t* __restrict__ offsets, int32_t* __restrict__ num_padded,
    int32_t* __restrict__ flags) {
  align_small_body([&](int t, int j) { return ids[(size_t)t * k + j]; }, T, k, E, bm_shift, cap,
                   sorted, tile_expert, offsets, num_padded, flags);
}

// Routing and grouping of a small batch in one launch (the decode regime,
// where every launch of the step counts; vLLM issue, section Problem: decode
// is bound by weight streaming and dispatch count).  Up to 16 tokens, so at
// most 256 pairs: each of the 16 waves routes one token (route_common.h) and
// keeps its ids in LDS; then per-expert counts by LDS atomics, the
// block_m-padded offsets by a block scan, each pair's rank inside its expert
// by counting the earlier pairs with the same id (pair ids ascend with the
// token, so this is the stable order), and per non-empty expert its tile
// entries and sentinels.  No per-wave expert masks: with this few pairs the
// mask clearing and per-expert popcounts of align_small_kernel (16 x E
// words) cost more than the grouping itself.
constexpr int kRouteAlignMaxT = kSmallWaves;

template <int EPL>
__global__ __launch_bounds__(kSmallT) void route_align_small_kernel(
    const float* __restrict__ logits, int T, int k, int E, int bm_shift, int cap,
    int32_t* __restrict__ ids, float* __restrict__ wts, int32_t* __restrict__ sorted,
    int32_t* __restrict__ tile_expert, int32_t* __restrict__ offsets,
    int32_t* __restrict__ num_padded, int32_t* __restrict__ flags) {
  __shared__ int s_ids[kRouteAlignMaxT * 16];
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_wave[kSmallWaves];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int P = T * k;
  const int bm = 1 << bm_shift;
  for (int e = tid; e < E; e += kSmallT) s_cnt[e] = 0;
  if (wave < T) {  // one token per wave
    int e;
    float w;
    rt::route_token<EPL>(logits + (size_t)wave * E, E, k, &e, &w);
    if (lane < k) {
      ids[(size_t)wave * k + lane] = e;
      wts[(size_t)wave * k + lane] = w;
      s_ids[wave * k + lane] = e;
    }
  }
  __syncthreads();
  const int my_e = tid < P ? s_ids[tid] : -1;  // the routing gives ids in [0, E)
  if (tid < P) atomicAdd(&s_cnt[my_e], 1);
  __syncthreads();
  const int tot = tid < E ? s_cnt[tid] : 0;
  const int pe = ((tot + bm - 1) >> bm_shift) << bm_shift;
  const int off = block_excl_scan(pe, s_wave);
  if (tid < E) {
    s_off[tid] = off;
    offsets[tid] = off;
  }
  if (tid == E - 1) {
    s_off[E] = off + pe;
    offsets[E] = off + pe;
    *num_padded = off + pe;
    *flags = 0;  // routed ids are in range and distinct within a token
  }
  __syncthreads();
  if (tid < P) {
    int rank = 0;
    for (int q = 0; q < tid; q++) rank += s_ids[q] == my_e;
    sorted[s_off[my_e] + rank] = tid;
  }
  if (tid < E && tot > 0) {
    const int o = s_off[tid], end = s_off[tid + 1];
    for (int i = o >> bm_shift; i < (end >> bm_shift); i++) tile_expert[i] = tid;
    for (int i = o + tot; i < end; i++) sorted[i] = P;
  }
  const int npad = s_off[E];
  for (int i = npad + tid; i < cap; i += kSmallT) sorted[i] = P;
  for (int i = (npad >> bm_shift) + tid; i < (cap >> bm_shift); i += kSmallT) tile_expert[i] = -1;
}

// count + scan + scatter in two launches for nchunks <= kPlaceMaxChunks:
// after align_count_kernel, every block of this launch reads the whole
// count matrix (E x nchunks ints, from L2), takes each expert's total and
// the pairs of the chunks before its own, and scans the padded totals
// itself; block 0 writes the expert offsets, num_padded and the flag word
// (the OR of the chunks' flags).  Blocks below nchunks then place their
// chunk's pairs (as align_scatter_kernel), and every block takes a share of
// the padding.
constexpr int kPlaceMaxChunks = 64;

__global__ __launch_bounds__(kChunk) void align_place_kernel(
    const int32_t* __restrict__ ids, int T, int k, int E, int nchunks, int bm_shift, int cap,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ chunk_flags,
    int32_t* __restrict__ sorted, int32_t* __restrict__ tile_expert,
    int32_t* __restrict__ offsets, int32_t* __restrict__ num_padded,
    int32_t* __restrict__ flags) {
  extern __shared__ unsigned long long mask[];  // [4][E]
  __shared__ int s_before[kMaxExperts];
  __shared__ int s_tot[kMaxExperts];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_wave[kChunk / 64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int P = T * k;
  const int own = blockIdx.x;  // the chunk this block places, if below nchunks
  const int t = own * kChunk + tid;
  const bool placing = own < nchunks;  // the same for the whole block
  const bool mine = placing && t < T;
  // This thread's token ids (up to kRegK of them kept in registers), loaded
  // before the count matrix so that both round trips overlap.
  constexpr int kRegK = 16;
  int te[kRegK];
#pragma unroll
  for (int j = 0; j < kRegK; j++) te[j] = mine && j < k ? ids[(size_t)t * k + j] : -1;
  if (placing)
    for (int i = tid; i < 4 * E; i += kChunk) mask[i] = 0ull;
  for (int e = tid; e < E; e += kChunk) {
    const int32_t* row = counts + (size_t)e * nchunks;
    int tot = 0, before = 0;
#pragma unroll 8
    for (int c = 0; c < nchunks; c++) {
      const int v = row[c];
      tot += v;
      before += c < own ? v : 0;
    }
    s_tot[e] = tot;
    s_before[e] = before;
  }
  __syncthreads();
  auto set_bit = [&](int e) __attribute__((always_inline)) {
    if (e >= 0 && e < E) atomicOr(&mask[wave * E + e], 1ull << lane);
  };
#pragma unroll
  for (int j = 0; j < kRegK; j++)
    if (mine && j < k) set_bit(te[j]);
  for (int j = kRegK; j < k; j++)
    if (mine) set_bit(ids[(size_t)t * k + j]);
  // Padded offsets: thread tid owns a contiguous run of experts.
  const int per = (E + kChunk - 1) / kChunk;
  const int r0 = min(E, tid * per), r1 = min(E, r0 + per);
  int run = 0;
  for (int e = r0; e < r1; e++) run += ((s_tot[e] + (1 << bm_shift) - 1) >> bm_shift) << bm_shift;
  int base = block_excl_scan(run, s_wave);
  for (int e = r0; e < r1; e++) {
    s_off[e] = base;
    base += ((s_tot[e] + (1 << bm_shift) - 1) >> bm_shift) << bm_shift;
  }
  if (tid == kChunk - 1) s_off[E] = base;
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int e = tid; e <= E; e += kChunk) offsets[e] = s_off[e];
    int bad = 0;
    for (int c = tid; c < nchunks; c += kChunk) bad |= chunk_flags[c];
    const int b1 = __syncthreads_or(bad & 1);
    const int b2 = __syncthreads_or(bad & 2);
    if (tid == 0) {
      *num_padded = s_off[E];
      *flags = (b1 ? 1 : 0) | (b2 ? 2 : 0);
    }
  }
  // Pair (t, j) goes to its expert's offset + the pairs of earlier chunks,
  // earlier waves and earlier lanes; j ascending, so a repeated id keeps the
  // later pair, as in the other paths.
  const unsigned long long below = (1ull << lane) - 1ull;
  auto place = [&](int e, int j) __attribute__((always_inline)) {
    if (e < 0 || e >= E) return;
    int rank = s_before[e] + __popcll(mask[wave * E + e] & below);
    for (int w = 0; w < wave; w++) rank += __popcll(mask[w * E + e]);
    sorted[s_off[e] + rank] = t * k + j;
  };
#pragma unroll
  for (int j = 0; j < kRegK; j++)
    if (mine && j < k) place(te[j], j);
  for (int j = kRegK; j < k; j++)
    if (mine) place(ids[(size_t)t * k + j], j);
  // Sentinels and tile entries: a group of block_m / 4 lanes per expert
  // (as in align_small_kernel).
  {
    const int gs_shift = bm_shift - 2;  // block_m is 16..128
    const int gs = 1 << gs_shift, per_wave = 64 >> gs_shift;
    const int sub = lane >> gs_shift, sl = lane & (gs - 1);
    const int ngroups = gridDim.x * (kChunk / 64) * per_wave;
    for (int e = (blockIdx.x * (kChunk / 64) + wave) * per_wave + sub; e < E; e += ngroups) {
      const int o = s_off[e], n = s_tot[e], end = s_off[e + 1];
      for (int i = (o >> bm_shift) + sl; i < (end >> bm_shift); i += gs) tile_expert[i] = e;
      for (int i = o + n + sl; i < end; i += gs) sorted[i] = P;
    }
  }
  const int npad = s_off[E];
  const int stride = gridDim.x * kChunk;
  for (int i = npad + blockIdx.x * kChunk + tid; i < cap; i += stride) sorted[i] = P;
  for (int i = (npad >> bm_shift) + blockIdx.x * kChunk + tid; i < (cap >> bm_shift);
       i += stride)
    tile_expert[i] = -1;
}

}  // namespace

hipError_t launch_align(const int32_t* ids, int T, int k, int E, int block_m, int32_t* sorted,
                        int32_t* tile_expert, int32_t* offsets, int32_t* num_padded,
                        int32_t* chunk_counts, int32_t* chunk_flags, int32_t* totals,
                        int32_t* flags, int cap, hipStream_t s) {
  if (E > kMaxExperts) return hipErrorInvalidValue;
  if (block_m < 16 || block_m > 128 || (block_m & (block_m - 1)) != 0) return hipErrorInvalidValue;
  const int nchunks = (T + kChunk - 1) / kChunk;
  const size_t lds = (size_t)4 * E * sizeof(unsigned long long);
  hipError_t err;
  // One block up to 512 tokens; beyond that the two-launch path measured
  // faster although the block could take 1024 (1024 tokens: 17.5 -> 14.0 us).
  constexpr int kSmallPathT = 512;
  static_assert(kSmallPathT <= kSmallT, "one thread per token");
  if (T <= kSmallPathT) {
    const int bm_shift = __builtin_ctz((unsigned)block_m);
    const size_t lds_small = (size_t)kSmallWaves * E * sizeof(unsigned long long);
    hipLaunchKernelGGL(align_small_kernel, dim3(1), dim3(kSmallT), lds_small, s, ids, T, k, E,
                       bm_shift, cap, sorted, tile_expert, offsets, num_padded, flags);
    return hipGetLastError();
  }
  if (nchunks > 0) {
    hipLaunchKernelGGL(align_count_kernel, dim3(nchunks), dim3(kChunk), lds, s, ids, T, k, E,
                       nchunks, chunk_counts, chunk_flags);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // At least 32 blocks share the padding writes even when there are few chunks.
  const int nblk = nchunks > 32 ? nchunks : 32;
  if (nchunks <= kPlaceMaxChunks) {
    hipLaunchKernelGGL(align_place_kernel, dim3(nblk), dim3(kChunk), lds, s, ids, T, k, E,
                       nchunks, __builtin_ctz((unsigned)block_m), cap, chunk_counts,
                       chunk_flags, sorted, tile_expert, offsets, num_padded, flags);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(align_scan_kernel, dim3(1), dim3(1024), 0, s, nchunks, E, block_m,
                     chunk_counts, totals, offsets, num_padded, chunk_flags, flags);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(align_scatter_kernel, dim3(nblk), dim3(kChunk), lds, s, ids, T, k, E,
                     nchunks, block_m, cap, chunk_counts, offsets, totals, sorted, tile_expert);
  return hipGetLastError();
}

size_t align_chunk_count(int T) { return (size_t)(T + kChunk - 1) / kChunk; }

int route_align_fused_max_tokens() { return kRouteAlignMaxT; }

hipError_t launch_route_align(const float* logits, int T, int E, int k, int block_m,
                              int32_t* ids, float* w, int32_t* sorted, int32_t* tile_expert,
                              int32_t* offsets, int32_t* num_padded, int32_t* flags, int cap,
                              hipStream_t s) {
  if (T < 1 || T > kRouteAlignMaxT || k > 16 || E > kMaxExperts) return hipErrorInvalidValue;
  if (block_m < 16 || block_m > 128 || (block_m & (block_m - 1)) != 0) return hipErrorInvalidValue;
  const int bm_shift = __builtin_ctz((unsigned)block_m);
#define QMOE_RA_CASE(EPL)                                                                   \
  if (E <= 64 * EPL) {                                                                      \
    hipLaunchKernelGGL(route_align_small_kernel<EPL>, dim3(1), dim3(kSmallT), 0, s,         \
                       logits, T, k, E, bm_shift, cap, ids, w, sorted, tile_expert, offsets, \
                       num_padded, flags);                                                  \
    return hipGetLastError();                                                               \
  }
  QMOE_RA_CASE(1)
  QMOE_RA_CASE(2)
  QMOE_RA_CASE(4)
  QMOE_RA_CASE(8)
  QMOE_RA_CASE(16)
#undef QMOE_RA_CASE
  return hipErrorInvalidValue;
}

}  // namespace qmoe
