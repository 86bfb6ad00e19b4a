// Stage 2 (down projection) of the grouped FFN with the tile's activation
// rows resident in LDS (aiter PR 6090, Test Plan: stage2 tiles; hip-ep PR
// "perf(qmoe): group prefill expert matmuls": one launch for every expert).
//
//   y_pairs[pair(row)] = hq[row] . W2[e]^T * s_h[row]
//
// For the schemes whose stage-2 activations are one byte (a8w4 fp8, W8A8
// int8), a row tile's quantized h rows (BM x I bytes, I <= 1024) fit in
// LDS.  A work item is (row tile, chunk of `passes` column passes of 256
// outputs): the block takes each row's scale s_h from the |h| maxima stage 1
// wrote per column tile, reads the tile's fp32 h rows once, quantizes them
// (the recipe of quant_common.h, the same codes a separate requantization
// pass gives) straight into LDS, then streams the expert's W2 rows for every
// pass of the chunk through a register ring that runs three K steps ahead
// across pass boundaries.  No barrier is needed between steps (the
// activations are read-only), and no activation row is loaded again.
//
// One block = 8 waves (two per SIMD), one block per CU; each wave owns two
// 16-column weight sub-tiles.  The MFMAs take the weight fragment as the A
// operand and the activation fragment as the B operand, so a lane's four
// accumulators are four consecutive output columns of one row, stored
// straight from registers (8 bytes of bf16, 16 bytes of fp32).  Operand
// layouts are the ones the row-major kernel uses (measured on gfx950: the
// fp4/fp8 pairing and the per-lane e8m0 scale routing do not depend on which
// operand slot holds which format).
#include "gemm_common.h"
#include "quant_common.h"

namespace qmoe {
namespace {

typedef float s2_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 s2_bf16x2 __attribute__((ext_vector_type(2)));

using namespace gk;

constexpr int kS2Waves = 8;
constexpr int kS2Threads = kS2Waves * 64;
constexpr int kS2Nsub = 2;
constexpr int kS2Cols = kS2Waves * kS2Nsub * 16;  // output columns per pass
constexpr int kS2RowBytes = 1024;                 // largest activation row held in LDS
// LDS row pitch: the 32-byte pad makes the 16-byte fragment reads (16 rows
// at 16q + 64f) free of bank conflicts on gfx950, measured.
constexpr int kS2Pitch = kS2RowBytes + 32;
constexpr int kS2MaxPasses = 16;  // W8A8: column passes whose weight scales sit in LDS

// One MFMA step with the weight fragment as the A operand.
template <int S>
__device__ inline void mfma_step_wa(typename Tr<S>::Acc& acc, const u32x4* a,
                                    const BFrag<S>& b) {
  if constexpr (S == kW8A8) {
#pragma unroll
    for (int j = 0; j < 2; j++)
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, b.q[j]),
                                                 __builtin_bit_cast(i32x4, a[j]), acc, 0, 0, 0);
  } else {
    // A = weights, fp4 (format 4) with the e8m0 byte of its 32-wide block
    // per lane (byte 0 for MFMA 0, byte 1 for MFMA 1); B = activations, fp8
    // (format 0) with unit scale.
    const i32x8 a0 = {(int)a[0].x, (int)a[0].y, (int)a[0].z, (int)a[0].w,
                      (int)a[1].x, (int)a[1].y, (int)a[1].z, (int)a[1].w};
    const i32x8 a1 = {(int)a[2].x, (int)a[2].y, (int)a[2].z, (int)a[2].w,
                      (int)a[3].x, (int)a[3].y, (int)a[3].z, (int)a[3].w};
    const i32x8 b0 = {(int)b.q[0].x, (int)b.q[0].y, (int)b.q[0].z, (int)b.q[0].w, 0, 0, 0, 0};
    const i32x8 b1 = {(int)b.q[1].x, (int)b.q[1].y, (int)b.q[1].z, (int)b.q[1].w, 0, 0, 0, 0};
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b0, a0, acc, 4, 0, 0, (int)b.sc, 0,
                                                           127);
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b1, a1, acc, 4, 0, 1, (int)b.sc, 0,
                                                           127);
  }
}

// SY: how each pass's outputs leave: 0 straight from registers; 1 (a8w4)
// staged in the free half of the activation rows' LDS slots (rows of at
// most half the slot; the launcher checks K); 2 staged 32 rows at a time in
// a buffer of their own (W8A8: tiles of up to 64 rows, no debug dump; the
// launcher checks both).
template <int S, int BM, bool PK, int SY>
__global__ __launch_bounds__(kS2Threads) __attribute__((amdgpu_waves_per_eu(2, 2))) void
moe_stage2_resident(GemmArgs g, int passes, int tile_div) {
  static_assert(S == kW8A8 || S == kA8W4, "one-byte activations only");
  static_assert(SY != 1 || S == kA8W4, "in-row staging holds bf16 outputs");
  static_assert(SY != 2 || S == kA8W4 || BM <= 64, "W8A8 staging fits LDS up to 64 rows");
  using T_ = Tr<S>;
  using Acc = typename T_::Acc;
  constexpr int MSUB = BM / 16;
  constexpr int NF = T_::A_FRAG / 16;
  __shared__ __attribute__((aligned(16))) uint8_t sA[BM * kS2Pitch];
  __shared__ __attribute__((aligned(16))) int sRow[BM];
  __shared__ __attribute__((aligned(16))) float sScale[BM];  // s_h of each row
  __shared__ __attribute__((aligned(16))) float sRcp[BM];    // RN(1 / s_h)
  __shared__ int sExpert;
  // W8A8: the item's per-channel weight scales (its columns are one
  // contiguous range of passes * kS2Cols), copied at the item's start so
  // that no pass epilogue waits on a global load behind the weight stream.
  __shared__ __attribute__((aligned(16))) float sWs[S == kW8A8 ? kS2MaxPasses * kS2Cols : 4];
  constexpr int kYEs = S == kA8W4 ? 2 : 4;  // output bytes per element
  constexpr int kYRows = 32, kYPitch = kS2Cols * kYEs + 16;
  __shared__ __attribute__((aligned(16))) uint8_t sY[SY == 2 ? kYRows * kYPitch : 16];
  __shared__ int sItem;  // the work item the block claimed from its XCD's queue

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int K = g.K;                     // = I; K bytes per activation row
  const int nsteps = K / T_::BK;
  const uint32_t kbytes = (uint32_t)(K * T_::KB_NUM / T_::KB_DEN);  // weight bytes per row
  const int num_m = *g.num_padded / BM;
  const int nchunk = g.ntiles_n / passes;
  const int total = num_m * nchunk;
  const int per_xcd = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int chunk = (total + 7) >> 3;
  const int w_begin = xcd * chunk, w_end = min(total, w_begin + chunk);
  const uint8_t* __restrict__ Aglob = reinterpret_cast<const uint8_t*>(g.a);
  // Fused quantization: g.a is stage 1's fp32 h and g.row_pmax its |h|
  // maxima; otherwise g.a holds the codes and g.a_scale the row scales.
  const bool fused = g.row_pmax != nullptr;
  const uint8_t* __restrict__ B = reinterpret_cast<const uint8_t*>(g.b);
  const uint32_t sshift = ((PK ? lane : lq) & 1) * 16;
  constexpr uint32_t B_KS = PK ? 16 * T_::B_STEP : T_::B_STEP;
  constexpr uint32_t B_PIECE = PK ? 1024 : 16;
  constexpr uint32_t S_KS = PK ? 128 : 8;
  constexpr int SB = 1;  // e8m0 bytes (a8w4); W8A8 scales are per channel
  const int G = passes * nsteps;  // weight steps of an item
  static_assert(kS2Cols * 2 <= kS2RowBytes / 2, "a pass's bf16 row piece fits the free half");

  Acc acc[MSUB][kS2Nsub];
  BFrag<S> b0[kS2Nsub], b1[kS2Nsub], b2[kS2Nsub], b3[kS2Nsub];

  // Work items: with g.queue, the blocks of an XCD claim the items of its
  // share one at a time from the XCD's counter (zeroed by stage 1, which
  // runs before this kernel on the same stream), so that a block that drew
  // short items (half tiles with few or no rows) takes more of them;
  // otherwise block `slot` takes every per_xcd-th item.  Every item writes
  // its own output rows, so the outputs do not depend on who took what.
  for (int it = 0;; it++) {
    if (g.queue != nullptr && tid == 0)
      sItem = w_begin + __hip_atomic_fetch_add(&g.queue[xcd], 1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();  // the previous item is done with sA / sRow / sScale; sItem is set
    const int wi = g.queue != nullptr ? sItem : w_begin + slot + it * per_xcd;
    if (wi >= w_end) break;
    const int mt = wi / nchunk, c = wi - mt * nchunk;
    int valid_here = 0;
    if (tid < BM) {
      const int p = g.sorted_pair_ids[mt * BM + tid];
      const bool ok = p < g.P;
      sRow[tid] = ok ? p : -1;
      // Row scale: the row's |h| max over stage 1's column tiles (fused
      // quantization), or the scale the requantization pass wrote.
      float a = 0.f;
      if (ok && fused) {
        const float* pm = g.row_pmax + ((size_t)mt * BM + tid) * g.pmax_stride;
        for (int i = 0; i < g.pmax_stride; i++) a = fmaxf(a, pm[i]);
      }
      const float sh = fused ? rq::row_scale<S == kA8W4>(a) : 1.0f;
      sScale[tid] = ok ? (fused ? sh : g.a_scale[(size_t)mt * BM + tid]) : 0.f;
      sRcp[tid] = ok ? 1.0f / sh : 0.f;
      valid_here = ok;
    }
    if (tid == kS2Threads - 1) sExpert = g.tile_expert[mt / tile_div];
    const int nvalid = __syncthreads_count(valid_here);
    if (nvalid == 0) continue;  // a part of a tile past its expert's last row
    const int mvalid = (nvalid + 15) >> 4;
    const int e = sExpert;
    if constexpr (S == kW8A8) {
      const float* ws = reinterpret_cast<const float*>(g.b_scale) + (size_t)e * g.N +
                        (size_t)c * passes * kS2Cols;
      for (int i = tid; i < passes * kS2Cols; i += kS2Threads) sWs[i] = ws[i];
    }

    // Weight cursor: the load for global step gs of this item reads column
    // pass gs / nsteps, K step gs % nsteps; steps past the item re-read its
    // last step (cache hits), so every step has the same shape.
    const uint8_t* __restrict__ Bexp = B + (size_t)e * g.N * kbytes;
    const uint8_t* __restrict__ Sexp =
        reinterpret_cast<const uint8_t*>(g.b_scale) + (size_t)e * g.N * (K / 32) * SB;
    auto load_b = [&](BFrag<S>(&bf)[kS2Nsub], int gs) __attribute__((always_inline)) {
      gs = min(gs, G - 1);
      const int p = gs / nsteps, ks = gs - p * nsteps;
      const int col0 = (c * passes + p) * kS2Cols + wave * kS2Nsub * 16;  // first weight row
#pragma unroll
      for (int s = 0; s < kS2Nsub; s++) {
        const uint32_t g16 = (uint32_t)(col0 + s * 16);
        uint32_t o, so;
        if constexpr (PK) {
          o = g16 * kbytes + lane * 16 + (uint32_t)ks * B_KS;
          so = g16 * (uint32_t)(K / 32) * SB + lane * 2 + (uint32_t)ks * S_KS;
        } else {
          o = (g16 + lr) * kbytes + lq * T_::B_FRAG + (uint32_t)ks * B_KS;
          so = (g16 + lr) * (uint32_t)(K / 32) * SB + lq * 2 + (uint32_t)ks * S_KS;
        }
#pragma unroll
        for (int i = 0; i < T_::B_FRAG / 16; i++)
          bf[s].q[i] = *reinterpret_cast<const u32x4*>(Bexp + (uint32_t)(o + B_PIECE * i));
        if constexpr (S == kA8W4)
          bf[s].sc = *reinterpret_cast<const uint32_t*>(Sexp + (so & ~3u));
        else
          bf[s].sc = 0;
      }
    };
    load_b(b0, 0);
    load_b(b1, 1);
    load_b(b2, 2);

    // The tile's h rows into LDS as codes.  Fused quantization: a thread
    // takes 16 consecutive values of a row (four 16-byte loads of fp32 h),
    // quantizes them with the row's scale and writes one 16-byte piece of
    // codes; kBatch pieces per thread are loaded before any is quantized.
    // Otherwise the requantization pass's codes are copied, eight 16-byte
    // pieces per thread in flight.  Rows past the tile's last real row, to
    // the end of its 16-row group, only feed discarded outputs and are
    // written as zeros.
    if (!fused) {
      constexpr int kBatch = 8;
      const int cpr = K / 16;  // 16-byte pieces per row
      const int n = mvalid * 16 * cpr;
      for (int i0 = tid; i0 < n; i0 += kBatch * kS2Threads) {
        u32x4 v[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; j++) {
          const int i = i0 + j * kS2Threads;
          const int r = i / cpr, cc = i - r * cpr;
          v[j] = u32x4{0u, 0u, 0u, 0u};
          if (i < n && r < nvalid)
            v[j] = *reinterpret_cast<const u32x4*>(Aglob + ((size_t)mt * BM + r) * (size_t)K +
                                                   cc * 16);
        }
#pragma unroll
        for (int j = 0; j < kBatch; j++) {
          const int i = i0 + j * kS2Threads;
          const int r = i / cpr, cc = i - r * cpr;
          if (i < n) *reinterpret_cast<u32x4*>(sA + r * kS2Pitch + cc * 16) = v[j];
        }
      }
    } else {
      constexpr int kBatch = 2;
      const int cpr = K / 16;  // 16-value pieces per row
      const int n = mvalid * 16 * cpr;
      const float* __restrict__ H32 = reinterpret_cast<const float*>(Aglob);
      for (int i0 = tid; i0 < n; i0 += kBatch * kS2Threads) {
        f32x4 v[kBatch][4];
#pragma unroll
        for (int j = 0; j < kBatch; j++) {
          const int i = i0 + j * kS2Threads;
          const int r = i / cpr, cc = i - r * cpr;
          if (i < n && r < nvalid) {
            const f32x4* src =
                reinterpret_cast<const f32x4*>(H32 + ((size_t)mt * BM + r) * K + cc * 16);
#pragma unroll
            for (int u = 0; u < 4; u++) v[j][u] = __builtin_nontemporal_load(src + u);
          }
        }
#pragma unroll
        for (int j = 0; j < kBatch; j++) {
          const int i = i0 + j * kS2Threads;
          const int r = i / cpr, cc = i - r * cpr;
          if (i < n) {
            u32x4 q = {0u, 0u, 0u, 0u};
            if (r < nvalid) {
              const float sh = sScale[r], rc = sRcp[r];
              const bool refine = sh >= 0x1p-60f;
#pragma unroll
              for (int u = 0; u < 4; u++)
                q[u] = rq::quant4<S == kA8W4>(v[j][u][0], v[j][u][1], v[j][u][2], v[j][u][3], sh,
                                              rc, refine);
            }
            *reinterpret_cast<u32x4*>(sA + r * kS2Pitch + cc * 16) = q;
          }
        }
      }
    }
#pragma unroll
    for (int m = 0; m < MSUB; m++)
#pragma unroll
      for (int s = 0; s < kS2Nsub; s++) acc[m][s] = Acc{0, 0, 0, 0};
    __syncthreads();

    auto read_frag = [&](u32x4(&af)[NF], int ks, int m) __attribute__((always_inline)) {
      const uint8_t* src = sA + (m * 16 + lr) * kS2Pitch + ks * T_::A_STEP;
#pragma unroll
      for (int f = 0; f < NF; f++)
        af[f] = *reinterpret_cast<const u32x4*>(src + a_frag_offset<S, PK>(lq, f));
    };
    auto compute = [&](int ks, const BFrag<S>(&bcr)[kS2Nsub]) __attribute__((always_inline)) {
      BFrag<S> bc[kS2Nsub];
#pragma unroll
      for (int s = 0; s < kS2Nsub; s++) {
        bc[s] = bcr[s];
        bc[s].sc = bcr[s].sc >> sshift;
      }
      u32x4 fa[NF], fb[NF];
      read_frag(fa, ks, 0);
#pragma unroll
      for (int m = 0; m < MSUB; m++) {
        if (m < mvalid) {
          if (m + 1 < MSUB && m + 1 < mvalid) read_frag((m & 1) ? fa : fb, ks, m + 1);
#pragma unroll
          for (int s = 0; s < kS2Nsub; s++) mfma_step_wa<S>(acc[m][s], (m & 1) ? fb : fa, bc[s]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // Outputs of column pass p: lane (lq, lr) holds, for row m*16 + lr,
    // the four columns 4*lq .. 4*lq+3 of each sub-tile.
    //
    // Staged: the pass's outputs go to LDS first, then every row's piece
    // (512 bytes of bf16, 1 KiB of fp32) leaves as 16-byte stores side by
    // side, instead of 32- or 64-byte pieces of 16 rows per store.
    auto epilogue_staged = [&](int p) __attribute__((always_inline)) {
      constexpr int kStage = kS2RowBytes / 2;
      constexpr int CH = SY == 2 ? (MSUB < kYRows / 16 ? MSUB : kYRows / 16) : MSUB;
      constexpr int kChunks = kS2Cols * kYEs / 16;  // 16-byte pieces of a row's pass
      auto stage_row = [&](int r) __attribute__((always_inline)) -> uint8_t* {
        if constexpr (SY == 2)
          return sY + (r % (CH * 16)) * kYPitch;
        else
          return sA + r * kS2Pitch + kStage;
      };
      const int col0 = (c * passes + p) * kS2Cols;
#pragma unroll
      for (int m0 = 0; m0 < MSUB; m0 += CH) {
        if (m0 < mvalid) {
          __syncthreads();  // the previous copy-out is done with the staging rows
#pragma unroll
          for (int mm = 0; mm < CH; mm++) {
            const int m = m0 + mm;
            if (m < mvalid) {
              const int row = m * 16 + lr;
              const float rs = sScale[row];
#pragma unroll
              for (int s = 0; s < kS2Nsub; s++) {
                const int cl = wave * kS2Nsub * 16 + s * 16 + 4 * lq;  // column in the pass
                if constexpr (S == kA8W4) {
                  const uint32_t lo = __builtin_bit_cast(
                      uint32_t,
                      __builtin_convertvector(
                          (s2_f32x2){acc[m][s][0] * rs, acc[m][s][1] * rs}, s2_bf16x2));
                  const uint32_t hi = __builtin_bit_cast(
                      uint32_t,
                      __builtin_convertvector(
                          (s2_f32x2){acc[m][s][2] * rs, acc[m][s][3] * rs}, s2_bf16x2));
                  *reinterpret_cast<uint2*>(stage_row(row) + cl * 2) = make_uint2(lo, hi);
                } else {
                  const float4 ws = *reinterpret_cast<const float4*>(&sWs[p * kS2Cols + cl]);
                  *reinterpret_cast<float4*>(stage_row(row) + cl * 4) =
                      make_float4(((float)acc[m][s][0] * rs) * ws.x,
                                  ((float)acc[m][s][1] * rs) * ws.y,
                                  ((float)acc[m][s][2] * rs) * ws.z,
                                  ((float)acc[m][s][3] * rs) * ws.w);
                }
                acc[m][s] = Acc{0, 0, 0, 0};
              }
            }
          }
          __syncthreads();
          const int r0 = m0 * 16, r1 = min(m0 + CH, mvalid) * 16;
          for (int i = tid; i < (r1 - r0) * kChunks; i += kS2Threads) {
            const int r = r0 + i / kChunks, ch = i % kChunks;
            const int pair = sRow[r];
            if (pair >= 0)
              *reinterpret_cast<u32x4*>(reinterpret_cast<uint8_t*>(g.out) +
                                        ((size_t)pair * g.H + col0) * kYEs + ch * 16) =
                  *reinterpret_cast<const u32x4*>(stage_row(r) + ch * 16);
          }
        }
      }
    };
    auto epilogue = [&](int p) __attribute__((always_inline)) {
      if constexpr (SY != 0) {
        epilogue_staged(p);
        return;
      }
      const int colw = (c * passes + p) * kS2Cols + wave * kS2Nsub * 16 + 4 * lq;
#pragma unroll
      for (int m = 0; m < MSUB; m++) {
        if (m < mvalid) {
          const int row = m * 16 + lr;
          const int pair = sRow[row];
          const float rs = sScale[row];
#pragma unroll
          for (int s = 0; s < kS2Nsub; s++) {
            const int col = colw + s * 16;
            if constexpr (S == kA8W4) {
              // Two values per conversion, each rounded to nearest even.
              const uint32_t lo = __builtin_bit_cast(
                  uint32_t, __builtin_convertvector(
                                (s2_f32x2){acc[m][s][0] * rs, acc[m][s][1] * rs}, s2_bf16x2));
              const uint32_t hi = __builtin_bit_cast(
                  uint32_t, __builtin_convertvector(
                                (s2_f32x2){acc[m][s][2] * rs, acc[m][s][3] * rs}, s2_bf16x2));
              if (pair >= 0)
                *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(g.out) +
                                          (size_t)pair * g.H + col) = make_uint2(lo, hi);
            } else {
              const float4 ws = *reinterpret_cast<const float4*>(
                  &sWs[p * kS2Cols + wave * kS2Nsub * 16 + 4 * lq + s * 16]);
              const float4 y = make_float4(((float)acc[m][s][0] * rs) * ws.x,
                                           ((float)acc[m][s][1] * rs) * ws.y,
                                           ((float)acc[m][s][2] * rs) * ws.z,
                                           ((float)acc[m][s][3] * rs) * ws.w);
              if (pair >= 0) {
                *reinterpret_cast<float4*>(reinterpret_cast<float*>(g.out) + (size_t)pair * g.H +
                                           col) = y;
                if (g.dump != nullptr)
                  *reinterpret_cast<int4*>(g.dump + ((size_t)mt * BM + row) * g.H + col) =
                      make_int4(acc[m][s][0], acc[m][s][1], acc[m][s][2], acc[m][s][3]);
              }
            }
            acc[m][s] = Acc{0, 0, 0, 0};
          }
        }
      }
    };

    // Step gs computes with weight register set gs % 4 and loads step gs+3
    // into the set that step gs-1 used.
    auto step = [&](int gs, const BFrag<S>(&bc)[kS2Nsub], BFrag<S>(&bl)[kS2Nsub])
        __attribute__((always_inline)) {
      load_b(bl, gs + 3);
      if (gs < G) {
        const int p = gs / nsteps, ks = gs - p * nsteps;
        compute(ks, bc);
        if (ks == nsteps - 1) epilogue(p);
      }
    };
    for (int gs = 0; gs < G; gs += 4) {
      step(gs, b0, b3);
      step(gs + 1, b1, b0);
      step(gs + 2, b2, b1);
      step(gs + 3, b3, b2);
    }
  }
}

template <int S, int BM, bool PK>
hipError_t launch_s2r(const GemmArgs& g, int passes, int tile_div, hipStream_t s) {
  int nblk = device_cu_count();
  nblk = nblk < 8 ? 8 : (nblk / 8) * 8;
  if constexpr (S == kA8W4) {
    if (g.K <= kS2RowBytes / 2)
      hipLaunchKernelGGL((moe_stage2_resident<S, BM, PK, 1>), dim3(nblk), dim3(kS2Threads), 0, s,
                         g, passes, tile_div);
    else
      hipLaunchKernelGGL((moe_stage2_resident<S, BM, PK, 2>), dim3(nblk), dim3(kS2Threads), 0, s,
                         g, passes, tile_div);
    return hipGetLastError();
  }
  if constexpr (BM <= 64) {
    if (g.dump == nullptr) {
      hipLaunchKernelGGL((moe_stage2_resident<S, BM, PK, 2>), dim3(nblk), dim3(kS2Threads), 0, s,
                         g, passes, tile_div);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((moe_stage2_resident<S, BM, PK, 0>), dim3(nblk), dim3(kS2Threads), 0, s, g,
                     passes, tile_div);
  return hipGetLastError();
}

// rows: the work item's rows (block_m, or half of it, tile_div = 2).
template <int S, bool PK>
hipError_t launch_s2r_bm(int rows, int tile_div, const GemmArgs& g, int passes,
                         hipStream_t s) {
  switch (rows) {
    case 16: return launch_s2r<S, 16, PK>(g, passes, tile_div, s);
    case 32: return launch_s2r<S, 32, PK>(g, passes, tile_div, s);
    case 64: return launch_s2r<S, 64, PK>(g, passes, tile_div, s);
    case 128: return launch_s2r<S, 128, PK>(g, passes, tile_div, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// W4A8 (scheme 3) takes the row-major stage 2 of gemm.hip: with the weights
// as the first operand its group scales would differ across a lane's four
// outputs.
bool stage2_resident_ok(int scheme, int I) {
  return (scheme == 1 || scheme == 2) && I <= kS2RowBytes;
}

int stage2_resident_cols() { return kS2Cols; }

int stage2_resident_max_passes(int scheme) { return scheme == 1 ? kS2MaxPasses : 1 << 30; }

hipError_t launch_stage2_resident(int scheme, int block_m, bool half_tiles, bool packed,
                                  const GemmArgs& g, int passes, hipStream_t s) {
  if (scheme == 1 && passes > kS2MaxPasses) return hipErrorInvalidValue;
  const int rows = half_tiles ? block_m / 2 : block_m, div = half_tiles ? 2 : 1;
  if (scheme == 2)
    return packed ? launch_s2r_bm<kA8W4, true>(rows, div, g, passes, s)
                  : launch_s2r_bm<kA8W4, false>(rows, div, g, passes, s);
  if (scheme == 1)
    return packed ? launch_s2r_bm<kW8A8, true>(rows, div, g, passes, s)
                  : launch_s2r_bm<kW8A8, false>(rows, div, g, passes, s);
  return hipErrorInvalidValue;
}

}  // namespace qmoe
