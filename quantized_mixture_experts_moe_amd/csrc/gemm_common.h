// Building blocks shared by the grouped-GEMM kernels (not installed): the
// per-scheme step geometry, weight fragments, the MFMA step of each scheme
// and the SiLU epilogue recipe.
#pragma once
#include <hip/hip_fp16.h>

#include "qmoe_internal.h"

namespace qmoe {
namespace gk {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
// Native 16-byte vector (HIP's uint4 is a struct, which keeps arrays of it
// out of registers).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

enum { kW4A16 = 0, kW8A8 = 1, kA8W4 = 2, kW4A8 = 3 };

// s_waitcnt immediate (gfx9 encoding) waiting for vmcnt == 0 only:
// vmcnt bits [3:0] and [15:14] = 0, expcnt [6:4] = 7, lgkmcnt [11:8] = 15.
constexpr int kWaitVmcnt0 = 0x0F70;

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

// W4A8: int8 activations x int4 weights, one v_mfma_i32_16x16x32_i8 per
// 32-wide scale group (its int32 result is the exact group sum, scaled once
// in fp32).  A step is 128 K = four groups; per MFMA j a lane holds 8 bytes
// of K [32j + 8q, +8) of its row (A) and of its column (B).
template <>
struct Tr<kW4A8> {
  static constexpr int BK = 128;
  static constexpr int A_ELEM = 1;
  static constexpr int A_STEP = 128;
  static constexpr int A_FRAG = 32;   // four 8-byte pieces per lane per 16-row group
  static constexpr int B_STEP = 64;   // int4 codes per row per step
  static constexpr int B_FRAG = 16;   // four 4-byte code words per lane per sub-tile
  static constexpr int KB_NUM = 1, KB_DEN = 2;
  typedef f32x4 Acc;
};

// Byte offset, inside a staged activation row of one step, of the f-th
// 16-byte piece of lane group q's A fragment (a8w4: pieces 2j, 2j+1 feed
// MFMA j; w8a8 and w4a16: piece j feeds MFMA j).  With the streaming weight
// layout every MFMA of a step covers one contiguous K range, so the pieces
// sit at 16q + 64f for the 8-bit schemes (a pattern free of LDS bank
// conflicts on gfx950, measured); the canonical layout keeps each lane's
// weight bytes contiguous and the A pieces follow it.
template <int S, bool PK>
__device__ inline int a_frag_offset(int q, int f) {
  if constexpr (PK && S != kW4A16) {
    return 16 * q + 64 * f;
  } else if constexpr (S == kA8W4) {
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
  uint32_t sc;   // w4a16: fp16 group scale bits; a8w4: two e8m0 bytes; w8a8: unused;
                 // w4a8: the fp16 scales of MFMAs 0 and 1
  uint32_t sc2;  // w4a8: the fp16 scales of MFMAs 2 and 3 (others: unused)
};

// Eight int4 codes (two's complement, element i in bits 4i..4i+3) times the
// group scale, each rounded once to bf16 (RNE).  With n = nibble ^ 8 = q + 8
// in 0..15, placing n into the fp16 pattern of 1024 gives the exact
// fp16 value 1024 + n (nibble in mantissa bits 0-3) or 1024 + 16n (bits
// 4-7), two per 32-bit word; a mixed-precision FMA then computes
//   (1024 + n) * s - 1032 s      = q * s,   or
//   (1024 + 16n) * (s/16) - 72 s = q * s,
// every product and constant exact in fp32 (at most 22 significant bits),
// so the only rounding is the final one to bf16: the same values as
// converting q and multiplying.  Per eight weights: one shift, four
// three-input bit operations, eight mixed FMAs and four bf16 packs.
__device__ inline bf16x8 dequant8_bf16(uint32_t v, float sc) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const uint32_t y = v >> 8;  // elements 2, 3, 6, 7 in the low nibbles
  const float s16 = sc * 0.0625f;
  const float c0 = -1032.0f * sc, c1 = -72.0f * sc;
  // One bit operation per pair: bit function 0x6A of (a, m, p) is
  // m ? a ^ p : p, so with m = the two nibbles and p = 0x6400 in each half
  // plus each nibble's bit 3, it gives ((a ^ 0x8888...) & m) | 0x64006400:
  // the nibbles with n = q + 8 (bit 3 flipped) inside the fp16 pattern.
  auto pair = [](uint32_t a, uint32_t m, uint32_t p) __attribute__((always_inline)) {
    return __builtin_bit_cast(f16x2, __builtin_amdgcn_bitop3_b32(a, m, p, 0x6A));
  };
  const f16x2 p04 = pair(v, 0x000F000Fu, 0x64086408u), p15 = pair(v, 0x00F000F0u, 0x64806480u);
  const f16x2 p26 = pair(y, 0x000F000Fu, 0x64086408u), p37 = pair(y, 0x00F000F0u, 0x64806480u);
  const float e0 = __builtin_fmaf((float)p04[0], sc, c0), e4 = __builtin_fmaf((float)p04[1], sc, c0);
  const float e1 = __builtin_fmaf((float)p15[0], s16, c1), e5 = __builtin_fmaf((float)p15[1], s16, c1);
  const float e2 = __builtin_fmaf((float)p26[0], sc, c0), e6 = __builtin_fmaf((float)p26[1], sc, c0);
  const float e3 = __builtin_fmaf((float)p37[0], s16, c1), e7 = __builtin_fmaf((float)p37[1], s16, c1);
  u32x4 w;
  w[0] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){e0, e1}, bf16x2));
  w[1] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){e2, e3}, bf16x2));
  w[2] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){e4, e5}, bf16x2));
  w[3] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){e6, e7}, bf16x2));
  return __builtin_bit_cast(bf16x8, w);
}

// A step's weight fragment in the form the MFMAs take: w4a16 dequantizes
// its int4 codes to bf16 once per step (the result is reused by every
// 16-row group of the tile); the 8-bit schemes feed the codes as they are.
template <int S>
struct BReady {
  BFrag<S> f;
};
template <>
struct BReady<kW4A16> {
  bf16x8 v[4];
};
// w4a8: per MFMA j the 8 int8 weights 16*q of K [32j + 8q, +8) in natural K
// order (w[2j]: K 0-3, w[2j+1]: K 4-7) and the group scale / 16.
template <>
struct BReady<kW4A8> {
  uint32_t w[8];
  float s[4];
};

// W4A8 unpacking: a nibble placed in the high half of a byte is the int8
// value 16*q exactly (two's complement), so (v << 4) & 0xF0F0F0F0 holds the
// low nibbles of v's four bytes and v & 0xF0F0F0F0 the high ones.  The
// streaming layout stores K b and b + 4 in byte b of each word (low, high
// nibble), which gives K 0-3 and 4-7 directly; the canonical layout stores K
// 2c and 2c + 1 in byte c, so two byte permutations interleave them.
template <bool PK>
__device__ inline void unpack_w4a8(uint32_t v, uint32_t& k03, uint32_t& k47) {
  const uint32_t lo = (v << 4) & 0xF0F0F0F0u, hi = v & 0xF0F0F0F0u;
  if constexpr (PK) {
    k03 = lo;
    k47 = hi;
  } else {
    // lo = K 0, 2, 4, 6 and hi = K 1, 3, 5, 7 (one byte each): interleave.
    k03 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
    k47 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
  }
}

// `sshift` (0 or 16) picks this lane's 16-bit scale field out of the
// aligned 32-bit word the weight loads fetch (w4a16, a8w4).
template <int S, bool PK = true>
__device__ inline BReady<S> prepare_b(const BFrag<S>& b, uint32_t sshift) {
  if constexpr (S == kW4A8) {
    BReady<S> r;
    const uint32_t words[4] = {b.q[0].x, b.q[0].y, b.q[0].z, b.q[0].w};
#pragma unroll
    for (int j = 0; j < 4; j++) unpack_w4a8<PK>(words[j], r.w[2 * j], r.w[2 * j + 1]);
    const uint32_t sw[2] = {b.sc, b.sc2};
#pragma unroll
    for (int j = 0; j < 4; j++)
      r.s[j] = __half2float(__ushort_as_half((unsigned short)(sw[j >> 1] >> (16 * (j & 1))))) *
               0.0625f;
    return r;
  } else if constexpr (S == kW4A16) {
    BReady<S> r;
    const float sc = __half2float(__ushort_as_half((unsigned short)(b.sc >> sshift)));
    r.v[0] = dequant8_bf16(b.q[0].x, sc);
    r.v[1] = dequant8_bf16(b.q[0].y, sc);
    r.v[2] = dequant8_bf16(b.q[0].z, sc);
    r.v[3] = dequant8_bf16(b.q[0].w, sc);
    return r;
  } else {
    BReady<S> r{b};
    r.f.sc = b.sc >> sshift;
    return r;
  }
}

template <int S>
__device__ inline void mfma_step(typename Tr<S>::Acc& acc, const u32x4* a, const BReady<S>& br) {
  if constexpr (S == kW4A16) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const bf16x8 av = __builtin_bit_cast(bf16x8, a[j]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, br.v[j], acc, 0, 0, 0);
    }
  } else if constexpr (S == kW8A8) {
    const BFrag<S>& b = br.f;
#pragma unroll
    for (int j = 0; j < 2; j++) {
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a[j]),
                                                 __builtin_bit_cast(i32x4, b.q[j]), acc, 0, 0, 0);
    }
  } else if constexpr (S == kW4A8) {
    // a[j >> 1] holds the 8-byte A pieces of MFMAs 2(j>>1) and 2(j>>1)+1.
    // Each MFMA starts from zero: its int32 result is 16 * the exact group
    // sum (|16 * sum| < 2^20, exact in fp32), scaled by s/16 in one fma.
    const i32x4 zero = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const u32x4 ap = a[j >> 1];
      const long av = (long)(((unsigned long)(j & 1 ? ap.w : ap.y) << 32) | (j & 1 ? ap.z : ap.x));
      const long bv = (long)(((unsigned long)br.w[2 * j + 1] << 32) | br.w[2 * j]);
      const i32x4 t = __builtin_amdgcn_mfma_i32_16x16x32_i8(av, bv, zero, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; r++) acc[r] = __builtin_fmaf((float)t[r], br.s[j], acc[r]);
    }
  } else {
    const BFrag<S>& b = br.f;
    // A fp8 (format 0) with unit scale 2^0 (e8m0 127); B fp4 (format 4) with
    // the e8m0 byte of its 32-wide block: byte 0 for MFMA 0, byte 1 for
    // MFMA 1.
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

// max(x, x of the lane that DPP control CTRL names); lanes of rows outside
// ROW_MASK keep x.
template <int CTRL, int ROW_MASK = 0xf>
__device__ inline float dpp_fmax(float x) {
  const int y = __builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, ROW_MASK,
                                            0xf, false);
  return fmaxf(x, __int_as_float(y));
}

// Maximum of x over each aligned group of G lanes (G = 16 or 32), exact in
// the group's last lane.  Four DPP steps reduce each 16-lane row (quad
// swaps, then the half-row and row mirrors); for G = 32 the last lane of
// the group's first row is then broadcast into its second row.
template <int G>
__device__ inline float group_max(float x) {
  static_assert(G == 16 || G == 32, "groups of 16 or 32 lanes");
  x = dpp_fmax<0xB1>(x);   // quad_perm [1,0,3,2]
  x = dpp_fmax<0x4E>(x);   // quad_perm [2,3,0,1]
  x = dpp_fmax<0x141>(x);  // row_half_mirror
  x = dpp_fmax<0x140>(x);  // row_mirror
  if constexpr (G == 32) x = dpp_fmax<0x142, 0xA>(x);  // row_bcast15 into rows 1 and 3
  return x;
}

// SiLU(gate) * up in the stage-1 epilogue.
// w8a8 follows the bit-exact fp32 recipe: ex = f32(exp_f64(-g));
// sg = g / (1 + ex) (IEEE division); h = sg * u.
// w4a16 and a8w4 use the hardware exp2 and reciprocal (a few ulp each; the
// library expf and IEEE division cost ~25 more instructions per element, a
// measured third of the tile epilogue):
// ex = exp2(-g * log2(e)); sg = g * rcp(1 + ex); h = sg * u.
template <int S>
__device__ inline float silu_mul(float g, float u) {
  if constexpr (S == kW8A8) {
    const float ex = (float)exp(-(double)g);
    const float den = 1.0f + ex;
    const float sg = g / den;
    return sg * u;
  } else {
    const float ex = __builtin_amdgcn_exp2f(-g * 1.44269504088896341f);
    const float sg = g * __builtin_amdgcn_rcpf(1.0f + ex);
    return sg * u;
  }
}

}  // namespace gk
}  // namespace qmoe
