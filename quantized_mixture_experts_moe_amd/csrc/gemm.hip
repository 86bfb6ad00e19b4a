// Grouped expert GEMMs: one launch per projection covers every expert (hip-ep
// PR "perf(qmoe): group prefill expert matmuls", description: expert
// projections batched into single launches instead of one per expert).
//
//   stage 1: gu = x[token(row)] . W13[e]^T, fused h = silu(gate) * up
//   stage 2: y_pairs[pair(row)] = h[row] . W2[e]^T
// (aiter PR 6090, Test Plan: stage1 tiles, then stage2 tiles.)
//
// Rows are the expert-sorted, block_m-padded pair slots from moe_align; a
// row tile never straddles two experts.  One workgroup = 8 waves (two per
// SIMD); each wave owns two 16-column weight sub-tiles (stage 1: the gate
// column and the up column of the same h column, so silu(gate)*up is formed
// in registers) and all BM rows.  Weight fragments stream from HBM straight
// into VGPRs, each weight byte read by exactly one wave, two K steps ahead of
// the MFMAs (a ring of three register sets); the gathered activation rows go
// global -> VGPR -> a three-slot LDS ring, loaded two steps ahead and shared
// by the 8 waves.  One barrier per K step.  16-row groups past the tile's
// last real row are skipped.
//
// Matrix cores (CDNA4 MFMA), 16x16 output per instruction:
//   w4a16: v_mfma_f32_16x16x32_bf16, int4 * fp16 group scale rounded to
//          bf16 in registers (the "dequantise then bf16 dot" lowering of the
//          vLLM issue "Evaluate native IU4/IU8 WMMA for grouped-INT MoE
//          prefill on gfx1151", section Constraint);
//   w8a8:  v_mfma_i32_16x16x64_i8, exact int32 accumulation (same issue,
//          section Constraint: integer products need int8 activations);
//   a8w4:  v_mfma_scale_f32_16x16x128_f8f6f4, A = fp8 e4m3, B = fp4 e2m1
//          with the e8m0 block scale fed per lane (aiter PR 6090, section
//          Changes: fp8 act, MXFP4 weight).
//
// Per-lane fragment layout of a 16x16xK MFMA (lane = 16*q + r): A row r and
// B column r hold a contiguous quarter q of the instruction's K (bf16, i8,
// and fp4 B of the scaled MFMA).  A step loads, per lane, a contiguous run of
// each weight row; the K order inside a step is permuted identically for A
// and B, which leaves the dot product unchanged, and every 32-wide scale
// block stays inside one lane.  One exception, measured on gfx950: with an
// fp8 A and an fp4 B the fp8 operand is split in two 16-byte halves, lane
// group q holding K [16q, 16q+16) in bytes 0-15 and K [64+16q, 64+16q+16)
// in bytes 16-31, while the fp4 B of lane group q covers K [32q, 32q+32)
// and takes that block's e8m0 scale from its own lane.  a_frag_offset()
// gathers the A bytes to match.
//
// Schedule: a persistent grid (a multiple of 8 blocks, one slice of the work
// list per XCD); work item = (row tile, column tile), row tile major, so the
// blocks of one XCD share the same gathered activation rows in their L2.
#include <hip/hip_fp16.h>

#include "qmoe_internal.h"

namespace qmoe {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
// Native 16-byte vector (HIP's uint4 is a struct, which keeps arrays of it
// out of registers).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

enum { kW4A16 = 0, kW8A8 = 1, kA8W4 = 2 };

template <int S>
struct Tr;
template <>
struct Tr<kW4A16> {
  static constexpr int BK = 128;      // K elements per pipeline step
  static constexpr int A_ELEM = 2;    // bytes per activation element (bf16)
  static constexpr int A_STEP = 256;  // activation bytes per row per step
  static constexpr int A_FRAG = 64;   // activation bytes per lane per 16-row group per step
  static constexpr int B_STEP = 64;   // weight bytes per row per step (int4)
  static constexpr int B_FRAG = 16;   // weight bytes per lane per sub-tile per step
  static constexpr int KB_NUM = 1, KB_DEN = 2;  // weight bytes per K element
  typedef f32x4 Acc;
};
template <>
struct Tr<kW8A8> {
  static constexpr int BK = 128;
  static constexpr int A_ELEM = 1;
  static constexpr int A_STEP = 128;
  static constexpr int A_FRAG = 32;
  static constexpr int B_STEP = 128;
  static constexpr int B_FRAG = 32;
  static constexpr int KB_NUM = 1, KB_DEN = 1;
  typedef i32x4 Acc;
};
template <>
struct Tr<kA8W4> {
  static constexpr int BK = 256;
  static constexpr int A_ELEM = 1;
  static constexpr int A_STEP = 256;
  static constexpr int A_FRAG = 64;
  static constexpr int B_STEP = 128;
  static constexpr int B_FRAG = 32;
  static constexpr int KB_NUM = 1, KB_DEN = 2;
  typedef f32x4 Acc;
};

// Byte offset, inside a staged activation row of one step, of the f-th
// 16-byte piece of lane group q's A fragment (pieces 2j, 2j+1 feed MFMA j).
template <int S>
__device__ inline int a_frag_offset(int q, int f) {
  if constexpr (S == kA8W4) {
    // B lane group q holds the 32-K blocks 2q (MFMA 0) and 2q+1 (MFMA 1) of
    // the 256-K step, so MFMA j's logical block b is step block 2b + j.  The
    // fp8 halves of lane group q map to logical K 16q and 64 + 16q.
    const int o = 64 * (q >> 1) + 16 * (q & 1);
    const int j = f >> 1, half = f & 1;
    return o + 32 * j + 128 * half;
  } else {
    return q * Tr<S>::A_FRAG + 16 * f;
  }
}

// Weight fragment of one 16-column sub-tile for one step.
template <int S>
struct BFrag {
  u32x4 q[Tr<S>::B_FRAG / 16];
  uint32_t sc;  // w4a16: fp16 group scale bits; a8w4: two e8m0 bytes; w8a8: unused
};

__device__ inline bf16x8 dequant8_bf16(uint32_t v, float sc) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int q = __builtin_amdgcn_sbfe((int)v, 4 * i, 4);  // two's-complement nibble
    r[i] = (__bf16)((float)q * sc);                          // exact product, one RNE rounding
  }
  return r;
}

template <int S>
__device__ inline void mfma_step(typename Tr<S>::Acc& acc, const u32x4* a, const BFrag<S>& b) {
  if constexpr (S == kW4A16) {
    const float sc = __half2float(__ushort_as_half((unsigned short)b.sc));
    const uint32_t w[4] = {b.q[0].x, b.q[0].y, b.q[0].z, b.q[0].w};
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const bf16x8 av = __builtin_bit_cast(bf16x8, a[j]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, dequant8_bf16(w[j], sc), acc, 0, 0, 0);
    }
  } else if constexpr (S == kW8A8) {
#pragma unroll
    for (int j = 0; j < 2; j++) {
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a[j]),
                                                 __builtin_bit_cast(i32x4, b.q[j]), acc, 0, 0, 0);
    }
  } else {
    // A fp8 (format 0) with unit scale 2^0 (e8m0 127); B fp4 (format 4) with
    // the e8m0 byte of its 32-wide block: byte 0 for the first 32 K of the
    // lane's run, byte 1 for the second.
    const i32x8 a0 = {(int)a[0].x, (int)a[0].y, (int)a[0].z, (int)a[0].w,
                      (int)a[1].x, (int)a[1].y, (int)a[1].z, (int)a[1].w};
    const i32x8 a1 = {(int)a[2].x, (int)a[2].y, (int)a[2].z, (int)a[2].w,
                      (int)a[3].x, (int)a[3].y, (int)a[3].z, (int)a[3].w};
    const i32x8 b0 = {(int)b.q[0].x, (int)b.q[0].y, (int)b.q[0].z, (int)b.q[0].w, 0, 0, 0, 0};
    const i32x8 b1 = {(int)b.q[1].x, (int)b.q[1].y, (int)b.q[1].z, (int)b.q[1].w, 0, 0, 0, 0};
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a0, b0, acc, 0, 4, 0, 127, 0,
                                                           (int)b.sc);
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a1, b1, acc, 0, 4, 0, 127, 1,
                                                           (int)b.sc);
  }
}

// fp32 epilogue recipe shared by w8a8 (bit-exact contract) and a8w4:
// ex = f32(exp_f64(-g)); sg = g / (1 + ex); h = sg * u.  w4a16 uses expf.
template <int S>
__device__ inline float silu_mul(float g, float u) {
  float ex;
  if constexpr (S == kW8A8) {
    ex = (float)exp(-(double)g);
  } else {
    ex = expf(-g);
  }
  const float den = 1.0f + ex;
  const float sg = g / den;
  return sg * u;
}

template <int S, int STAGE, int BM, int BPRE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void
moe_gemm_kernel(GemmArgs g) {
  using T_ = Tr<S>;
  using Acc = typename T_::Acc;
  constexpr int MSUB = BM / 16;
  constexpr int PITCH = T_::A_STEP + 16;                     // LDS row pitch (bytes), padded
  constexpr int CPR = T_::A_STEP / 16;                       // 16-byte chunks per row per step
  constexpr int NCH = (BM * CPR + kThreads - 1) / kThreads;  // chunks per thread per step
  constexpr int NF = T_::A_FRAG / 16;                        // 16-byte LDS reads per fragment
  constexpr int HALF = kNsub / 2;                            // stage 1: gate sub-tiles per wave

  __shared__ __attribute__((aligned(16))) uint8_t sA[kStages][BM * PITCH];
  __shared__ int sRow[BM];
  __shared__ float sRed[kWaves][BM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int num_m = *g.num_padded / BM;
  const int total = num_m * g.ntiles_n;
  const int per_xcd = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int chunk = (total + 7) >> 3;
  const int w_begin = xcd * chunk, w_end = min(total, w_begin + chunk);

  const size_t K = (size_t)g.K;
  const size_t kbytes = K * T_::KB_NUM / T_::KB_DEN;  // weight bytes per row
  const int nsteps = g.K / T_::BK;
  const uint8_t* __restrict__ A = reinterpret_cast<const uint8_t*>(g.a);
  const uint8_t* __restrict__ B = reinterpret_cast<const uint8_t*>(g.b);

  for (int wi = w_begin + slot; wi < w_end; wi += per_xcd) {
    const int mt = wi / g.ntiles_n, nt = wi - mt * g.ntiles_n;
    __syncthreads();  // previous tile is done with sA / sRow / sRed
    int valid_here = 0;
    if (tid < BM) {
      const int p = g.sorted_pair_ids[mt * BM + tid];
      const bool ok = p < g.P;
      sRow[tid] = ok ? (STAGE == 1 ? p / g.k : p) : -1;
      valid_here = ok;
    }
    const int nvalid = __syncthreads_count(valid_here);
    const int mvalid = (nvalid + 15) >> 4;
    const int e = g.tile_expert[mt];

    // Weight rows of this wave's sub-tiles, as 32-bit offsets from the
    // expert's base (one expert's weights are far below 4 GiB).
    int nrow[kNsub];
#pragma unroll
    for (int s = 0; s < kNsub; s++) {
      if (STAGE == 1) {
        const int base = nt * kStage1Cols + wave * HALF * 16 + lr;
        nrow[s] = s < HALF ? base + s * 16 : g.I + base + (s - HALF) * 16;
      } else {
        nrow[s] = nt * kStage2Cols + wave * kNsub * 16 + s * 16 + lr;
      }
    }
    constexpr int SB = S == kW4A16 ? 2 : 1;  // scale bytes (w4a16 fp16, a8w4 e8m0)
    const uint8_t* __restrict__ Bexp = B + (size_t)e * g.N * kbytes;
    const uint8_t* __restrict__ Sexp =
        reinterpret_cast<const uint8_t*>(g.b_scale) + (size_t)e * g.N * (K / 32) * SB;
    uint32_t boff[kNsub], soff[kNsub];
#pragma unroll
    for (int s = 0; s < kNsub; s++) {
      boff[s] = (uint32_t)nrow[s] * (uint32_t)kbytes + lq * T_::B_FRAG;
      soff[s] = (uint32_t)nrow[s] * (uint32_t)(K / 32) * SB + lq * 2;
    }

    auto load_b = [&](BFrag<S>(&bf)[kNsub], int ks) __attribute__((always_inline)) {
#pragma unroll
      for (int s = 0; s < kNsub; s++) {
        const u32x4* p =
            reinterpret_cast<const u32x4*>(Bexp + boff[s] + (uint32_t)ks * T_::B_STEP);
#pragma unroll
        for (int i = 0; i < T_::B_FRAG / 16; i++) bf[s].q[i] = p[i];
        if (S == kW4A16 || S == kA8W4)
          bf[s].sc = *reinterpret_cast<const unsigned short*>(Sexp + soff[s] + (uint32_t)ks * 8);
        else
          bf[s].sc = 0;
      }
    };

    // Activation chunks of this thread: fixed rows per tile.  Rows past the
    // tile's last real row read that row again (their results are dropped),
    // so every load is in bounds without a branch.
    uint32_t aoff[NCH];
#pragma unroll
    for (int i = 0; i < NCH; i++) {
      const int c = min(tid + i * kThreads, BM * CPR - 1);
      const int row = min(c / CPR, nvalid - 1), col = c % CPR;
      const uint32_t rbase = STAGE == 1 ? (uint32_t)sRow[row] * (uint32_t)(g.H * T_::A_ELEM)
                                        : (uint32_t)(mt * BM + row) * (uint32_t)(g.I * T_::A_ELEM);
      aoff[i] = rbase + col * 16;
    }
    u32x4 areg[NCH];
    auto load_a = [&](int ks) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < NCH; i++)
        areg[i] = *reinterpret_cast<const u32x4*>(A + aoff[i] + (uint32_t)ks * T_::A_STEP);
    };
    auto store_a = [&](int stage) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < NCH; i++) {
        const int c = tid + i * kThreads;
        const int row = c / CPR, col = c - row * CPR;
        if (NCH * kThreads == BM * CPR || c < BM * CPR)
          *reinterpret_cast<u32x4*>(&sA[stage][row * PITCH + col * 16]) = areg[i];
      }
    };

    Acc acc[MSUB][kNsub];
#pragma unroll
    for (int m = 0; m < MSUB; m++)
#pragma unroll
      for (int s = 0; s < kNsub; s++) acc[m][s] = Acc{0, 0, 0, 0};

    // Activation fragments are read from LDS one 16-row group ahead of the
    // MFMAs that use them; the scheduling fences keep the compiler from
    // hoisting every group's reads (which would need ~8x the registers).
    auto read_frag = [&](u32x4(&af)[NF], int stage, int m) __attribute__((always_inline)) {
      const uint8_t* src = &sA[stage][(m * 16 + lr) * PITCH];
#pragma unroll
      for (int f = 0; f < NF; f++)
        af[f] = *reinterpret_cast<const u32x4*>(src + a_frag_offset<S>(lq, f));
    };
    auto compute = [&](int stage, const BFrag<S>(&bc)[kNsub]) __attribute__((always_inline)) {
      u32x4 fa[NF], fb[NF];
      read_frag(fa, stage, 0);
#pragma unroll
      for (int m = 0; m < MSUB; m++) {
        if (m < mvalid) {
          if (m + 1 < MSUB && m + 1 < mvalid) read_frag((m & 1) ? fa : fb, stage, m + 1);
#pragma unroll
          for (int s = 0; s < kNsub; s++) mfma_step<S>(acc[m][s], (m & 1) ? fb : fa, bc[s]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // K loop: step s computes from LDS slot s%3, while the activation rows
    // of step s+1 are written to LDS and those of step s+2 are in flight.
    // Weights are loaded BPRE steps ahead into a ring of BPRE+1 register sets.
    const int n = nsteps;
    load_a(0);
    store_a(0);
    if (n > 1) load_a(1);
    if constexpr (BPRE == 2) {
      BFrag<S> b0[kNsub], b1[kNsub], b2[kNsub];
      auto step = [&](int s, const BFrag<S>(&bc)[kNsub], BFrag<S>(&bl)[kNsub]) __attribute__((always_inline)) {
        if (s >= n) return;
        if (s + 1 < n) store_a((s + 1) % kStages);
        if (s + 2 < n) {
          load_a(s + 2);
          load_b(bl, s + 2);
        }
        __syncthreads();
        compute(s % kStages, bc);
      };
      load_b(b0, 0);
      if (n > 1) load_b(b1, 1);
      for (int s = 0; s < n; s += 3) {
        step(s, b0, b2);
        step(s + 1, b1, b0);
        step(s + 2, b2, b1);
      }
    } else {
      BFrag<S> b0[kNsub], b1[kNsub];
      auto step = [&](int s, const BFrag<S>(&bc)[kNsub], BFrag<S>(&bl)[kNsub]) __attribute__((always_inline)) {
        if (s >= n) return;
        if (s + 1 < n) {
          store_a((s + 1) % kStages);
          load_b(bl, s + 1);
        }
        if (s + 2 < n) load_a(s + 2);
        __syncthreads();
        compute(s % kStages, bc);
      };
      load_b(b0, 0);
      for (int s = 0; s < n; s += 2) {
        step(s, b0, b1);
        step(s + 1, b1, b0);
      }
    }

    // ------------------------------------------------------------ epilogue
    if (STAGE == 1) {
      const float* ws = S == kW8A8 ? reinterpret_cast<const float*>(g.b_scale) + (size_t)e * g.N
                                   : nullptr;
      float amax[MSUB][4];
#pragma unroll
      for (int m = 0; m < MSUB; m++)
#pragma unroll
        for (int r = 0; r < 4; r++) amax[m][r] = 0.f;
#pragma unroll
      for (int s = 0; s < HALF; s++) {
        const int col = nrow[s];
        float ws_g = 1.f, ws_u = 1.f;
        if (S == kW8A8) {
          ws_g = ws[col];
          ws_u = ws[g.I + col];
        }
#pragma unroll
        for (int m = 0; m < MSUB; m++) {
          if (m < mvalid) {
#pragma unroll
            for (int r = 0; r < 4; r++) {
              const int row = m * 16 + lq * 4 + r;
              const int tok = sRow[row];
              const size_t orow = (size_t)mt * BM + row;
              float gf, uf;
              if constexpr (S == kW8A8) {
                const float xs = tok >= 0 ? g.a_scale[tok] : 0.f;
                gf = ((float)acc[m][s][r] * xs) * ws_g;
                uf = ((float)acc[m][s + HALF][r] * xs) * ws_u;
                if (g.dump != nullptr && tok >= 0) {
                  g.dump[orow * 2 * g.I + col] = acc[m][s][r];
                  g.dump[orow * 2 * g.I + g.I + col] = acc[m][s + HALF][r];
                }
              } else if constexpr (S == kA8W4) {
                const float xs = tok >= 0 ? g.a_scale[tok] : 0.f;
                gf = acc[m][s][r] * xs;
                uf = acc[m][s + HALF][r] * xs;
              } else {
                gf = acc[m][s][r];
                uf = acc[m][s + HALF][r];
              }
              const float h = tok >= 0 ? silu_mul<S>(gf, uf) : 0.f;
              if constexpr (S == kW4A16) {
                if (tok >= 0) reinterpret_cast<__bf16*>(g.out)[orow * g.I + col] = (__bf16)h;
              } else {
                if (tok >= 0) reinterpret_cast<float*>(g.out)[orow * g.I + col] = h;
                amax[m][r] = fmaxf(amax[m][r], fabsf(h));
              }
            }
          }
        }
      }
      if constexpr (S != kW4A16) {
#pragma unroll
        for (int m = 0; m < MSUB; m++) {
          if (m < mvalid) {
#pragma unroll
            for (int r = 0; r < 4; r++) {
              float a = amax[m][r];
#pragma unroll
              for (int off = 1; off < 16; off <<= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
              if (lr == 0) sRed[wave][m * 16 + lq * 4 + r] = a;
            }
          }
        }
        __syncthreads();
        if (tid < mvalid * 16) {
          float a = sRed[0][tid];
#pragma unroll
          for (int w = 1; w < kWaves; w++) a = fmaxf(a, sRed[w][tid]);
          g.row_pmax[((size_t)mt * BM + tid) * g.ntiles_n + nt] = a;
        }
      }
    } else {
#pragma unroll
      for (int s = 0; s < kNsub; s++) {
        const int col = nrow[s];
        float ws2 = 1.f;
        if (S == kW8A8) ws2 = reinterpret_cast<const float*>(g.b_scale)[(size_t)e * g.N + col];
#pragma unroll
        for (int m = 0; m < MSUB; m++) {
          if (m < mvalid) {
#pragma unroll
            for (int r = 0; r < 4; r++) {
              const int row = m * 16 + lq * 4 + r;
              const int pair = sRow[row];
              if (pair < 0) continue;
              const size_t orow = (size_t)mt * BM + row;
              if constexpr (S == kW8A8) {
                const float y = ((float)acc[m][s][r] * g.a_scale[orow]) * ws2;
                reinterpret_cast<float*>(g.out)[(size_t)pair * g.H + col] = y;
                if (g.dump != nullptr) g.dump[orow * g.H + col] = acc[m][s][r];
              } else if constexpr (S == kA8W4) {
                const float y = acc[m][s][r] * g.a_scale[orow];
                reinterpret_cast<__bf16*>(g.out)[(size_t)pair * g.H + col] = (__bf16)y;
              } else {
                reinterpret_cast<__bf16*>(g.out)[(size_t)pair * g.H + col] = (__bf16)acc[m][s][r];
              }
            }
          }
        }
      }
    }
  }
}

template <int S, int STAGE, int BM, int BPRE = 2>
hipError_t launch_one(const GemmArgs& g, hipStream_t s) {
  static int blocks_per_cu = 0;
  if (blocks_per_cu == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, moe_gemm_kernel<S, STAGE, BM, BPRE>, kThreads,
                                                     0) != hipSuccess ||
        n < 1)
      n = 1;
    blocks_per_cu = n;
  }
  int nblk = device_cu_count() * blocks_per_cu;
  nblk = nblk < 8 ? 8 : (nblk / 8) * 8;
  hipLaunchKernelGGL((moe_gemm_kernel<S, STAGE, BM, BPRE>), dim3(nblk), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

template <int S, int STAGE>
hipError_t launch_bm(int block_m, const GemmArgs& g, hipStream_t s) {
  switch (block_m) {
    case 16: return launch_one<S, STAGE, 16>(g, s);
    case 32: return launch_one<S, STAGE, 32>(g, s);
    case 64: return launch_one<S, STAGE, 64>(g, s);
    case 128: return launch_one<S, STAGE, 128>(g, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gemm(int scheme, int stage, int block_m, const GemmArgs& g, hipStream_t s) {
  switch (scheme * 2 + (stage - 1)) {
    case 0: return launch_bm<kW4A16, 1>(block_m, g, s);
    case 1: return launch_bm<kW4A16, 2>(block_m, g, s);
    case 2: return launch_bm<kW8A8, 1>(block_m, g, s);
    case 3: return launch_bm<kW8A8, 2>(block_m, g, s);
    case 4: return launch_bm<kA8W4, 1>(block_m, g, s);
    case 5: return launch_bm<kA8W4, 2>(block_m, g, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qmoe
