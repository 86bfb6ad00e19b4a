// Grouped expert GEMMs: one launch per projection covers every expert (hip-ep
// PR "perf(qmoe): group prefill expert matmuls", description: expert
// projections batched into single launches instead of one per expert).
//
//   stage 1: gu = x[token(row)] . W13[e]^T, fused h = silu(gate) * up
//   stage 2: y_pairs[pair(row)] = h[row] . W2[e]^T
// (aiter PR 6090, Test Plan: stage1 tiles, then stage2 tiles.)
//
// Rows are the expert-sorted, block_m-padded pair slots from moe_align; a
// row tile never straddles two experts.  One workgroup = 4 waves (one per
// SIMD, two workgroups per CU) or 8 waves (two per SIMD, one workgroup per
// CU); each wave owns two 16-column weight sub-tiles (stage 1: the gate
// column and the up column of the same h column, so silu(gate)*up is formed
// in registers) and all BM rows.  Weight fragments stream from HBM straight
// into VGPRs, each weight byte read by exactly one wave, RING-1 K steps
// ahead of the MFMAs (a ring of RING register sets: 8 for tiles of up to 32
// rows, 4 for taller ones); the gathered activation rows
// go global -> VGPR -> a two-slot LDS ring, loaded two steps ahead and
// shared by the block's waves.  One barrier per K step.  16-row groups past
// the tile's last real row are skipped.
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
//          Changes: fp8 act, MXFP4 weight);
//   w4a8:  v_mfma_i32_16x16x32_i8, int4 weights upconverted to int8 in
//          registers (vLLM issue, section Constraint: W4A8 with upconversion
//          of weights to IU8 before the MMA), one MFMA per 32-wide scale
//          group, its exact int32 sum scaled by the group scale in fp32.
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
// Schedule: a persistent grid (a multiple of 8 blocks, one share of the work
// list per XCD: a contiguous slice, or every eighth row tile where tiles of
// very different fill would leave some XCDs idle); work item = (row tile,
// column tile), row tile major, so the blocks of one XCD share the same
// gathered activation rows in their L2.
// Between the tiles of a block the stream of loads does not stop: in stage 1
// (K steps a multiple of four) the K loop's last three steps issue the next
// tile's first activation and weight loads, and the epilogue runs while they
// are in flight.
#include "gemm_common.h"

namespace qmoe {
namespace {

using namespace gk;


template <int S, int STAGE, int BM, bool PK, int NSUB, int WAVES, bool XT, int RING, bool LB>
__global__ __launch_bounds__(WAVES * 64)
    __attribute__((amdgpu_waves_per_eu(NSUB == 4 ? 1 : 2, NSUB == 4 ? 1 : 2))) void
    moe_gemm_kernel(GemmArgs g) {
  constexpr int kThreads = WAVES * 64;
  using T_ = Tr<S>;
  using Acc = typename T_::Acc;
  constexpr int MSUB = BM / 16;
  // LDS row pitch (bytes).  With a 32-byte pad the fragment reads of the
  // 8-bit schemes (16 rows x 16 bytes at 16q + 64f) reach 64 distinct banks
  // per 16 lanes: 4 LDS cycles per read instead of 8 with a 16-byte pad
  // (measured on gfx950).  w4a16's 64q + 16f pattern takes 8 cycles with
  // either pad.
  constexpr int PITCH = T_::A_STEP + (S == kW4A16 ? 16 : 32);
  constexpr int CPR = T_::A_STEP / 16;                       // 16-byte chunks per row per step
  constexpr int NCH = (BM * CPR + kThreads - 1) / kThreads;  // chunks per thread per step
  constexpr int NF = T_::A_FRAG / 16;                        // 16-byte LDS reads per fragment
  constexpr int HALF = NSUB / 2;                             // stage 1: gate sub-tiles per wave

  // Epilogue tile: the block's BM x COLS outputs, staged in LDS so that
  // global stores are 16 contiguous bytes per lane.  It lies over the
  // activation ring; with XT (next tile's first loads issued from the K
  // loop's last steps) it starts at ring slot 1, since slot 0 then already
  // holds the next tile's first activation step.
  constexpr int COLS = stage_cols(STAGE, NSUB, WAVES);
  constexpr int OUT_ES = STAGE == 1 ? (S == kW4A16 ? 2 : 4) : (S == kW8A8 ? 4 : 2);
  constexpr int EPITCH = COLS * OUT_ES + 16;
  constexpr int SLOT = BM * PITCH;
  constexpr int A_RING = kStages * SLOT;  // activation ring bytes
  constexpr int EPI = BM * EPITCH;
  constexpr int EPI_OFF = XT ? SLOT : 0;
  constexpr int SMEM = XT ? SLOT + (EPI > SLOT ? EPI : SLOT) : (A_RING > EPI ? A_RING : EPI);
  static_assert(kStages == 2, "two activation slots");
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
  uint8_t* const etile = smem + EPI_OFF;
  // Row ids of the tile being set up and of the tile in its epilogue.
  __shared__ __attribute__((aligned(16))) int sRow[2][BM];
  __shared__ __attribute__((aligned(16))) float sScale[BM];
  __shared__ int sExpert[2];
  auto sA = [&](int stage) __attribute__((always_inline)) { return smem + stage * BM * PITCH; };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int num_m = *g.num_padded / BM;
  const int per_xcd = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  // Work items of this XCD and the order in which this block takes them
  // (valid(u): the block has a u-th item; decode(u): its row and column
  // tile):
  //  - schedule 0: an even share of the row-tile-major item list, the
  //    blocks of the XCD strided over it;
  //  - schedule 1 (runs): an even share of the row tiles; the blocks of the
  //    XCD are split into groups of ntiles_n, block j of a group keeps
  //    column tile j, and the groups take contiguous runs of row tiles, so
  //    a block's consecutive items are consecutive row tiles of one column
  //    tile: when they belong to the same expert the second one reads the
  //    weights the first has just read (memory-side cache hits).  Taken
  //    only when per_xcd is a multiple of ntiles_n (schedule 0 otherwise);
  //  - schedule 2 (dealt row tiles): the XCD takes every eighth row tile
  //    (m = xcd, xcd + 8, ...) with all its column tiles, the blocks of the
  //    XCD strided over that list.  A row tile's activation rows still stay
  //    on one XCD, and each XCD gets the same mix of full and partial tiles:
  //    with skewed routing the contiguous shares of schedule 0 leave the
  //    XCDs that hold the rarely routed experts' short tiles idle for the
  //    last third of the kernel.
  // Schedules 0 and 2 share one form: item w of the XCD's list
  // [w_begin, w_end) is row tile m0 + mstep * (w / ntiles_n), column tile
  // w % ntiles_n.
  const bool dealt = g.schedule == 2;
  const int total = dealt ? (num_m > xcd ? (num_m - xcd + 7) >> 3 : 0) * g.ntiles_n
                          : num_m * g.ntiles_n;
  const int ichunk = dealt ? total : (total + 7) >> 3;
  const int w_begin = dealt ? 0 : min(total, xcd * ichunk);
  const int w_end = min(total, w_begin + ichunk);
  const int m0 = dealt ? xcd : 0, mstep = dealt ? 8 : 1;
  const int mchunk = (num_m + 7) >> 3;
  const int m_begin = min(num_m, xcd * mchunk), nm = min(num_m, m_begin + mchunk) - m_begin;
  const bool runs = g.schedule == 1 && per_xcd % g.ntiles_n == 0;  // else schedule 0 or 2
  const int groups = per_xcd / g.ntiles_n, grp = slot / g.ntiles_n;
  const int run_nt = slot - grp * g.ntiles_n;
  const int run_begin = grp < groups ? (int)((long)grp * nm / groups) : nm;
  const int run_end = grp < groups ? (int)((long)(grp + 1) * nm / groups) : nm;
  auto valid = [&](int u) __attribute__((always_inline)) {
    return runs ? run_begin + u < run_end : w_begin + slot + u * per_xcd < w_end;
  };
  auto decode = [&](int u, int& mt_out, int& nt_out) __attribute__((always_inline)) {
    if (runs) {
      mt_out = m_begin + run_begin + u;
      nt_out = run_nt;
    } else {
      const int w = w_begin + slot + u * per_xcd;
      const int r = w / g.ntiles_n;
      mt_out = m0 + mstep * r;
      nt_out = w - r * g.ntiles_n;
    }
  };

  static_assert(kThreads % CPR == 0, "chunk rows must be thread-invariant");
  static_assert(BM < kThreads, "the last thread loads the tile's expert id");
  const int lds_w = (tid / CPR) * PITCH + (tid % CPR) * 16;  // this thread's LDS store slot
  const size_t K = (size_t)g.K;
  const size_t kbytes = K * T_::KB_NUM / T_::KB_DEN;  // weight bytes per row
  const int nsteps = g.K / T_::BK;
  const uint8_t* __restrict__ A = reinterpret_cast<const uint8_t*>(g.a);
  const uint8_t* __restrict__ B = reinterpret_cast<const uint8_t*>(g.b);

  // Tile metadata (pair ids of the rows, the expert) is fetched one tile
  // ahead of the tile's set-up.
  // The tile's expert id is the same for the whole block, but it is loaded
  // by one thread only (the last one, never a row thread) and passed on
  // through LDS at the set-up barrier: a uniform load would be moved to a
  // scalar register right away, waiting for every load in flight.
  int next_pair = g.P, next_expert = 0, next_ri = -1;
  auto fetch_meta = [&](int u) __attribute__((always_inline)) {
    if (valid(u)) {
      int m, nt_unused;
      decode(u, m, nt_unused);
      if (tid < BM) next_pair = g.sorted_pair_ids[m * BM + tid];
      if (tid == kThreads - 1) next_expert = g.tile_expert[m];
    }
  };
  // Row id of a fetched pair slot (stage 1: its token), -1 for padding.  Run
  // right after a full wait for loads, so that the division (and a register
  // reload, if any) never waits inside the pipelined loop.
  auto decode_meta = [&]() __attribute__((always_inline)) {
    if (tid < BM) next_ri = next_pair < g.P ? (STAGE == 1 ? next_pair / g.k : next_pair) : -1;
  };

  // scale bytes (w4a16 and w4a8 fp16, a8w4 e8m0)
  constexpr int SB = (S == kW4A16 || S == kW4A8) ? 2 : 1;
  constexpr uint32_t B_KS = PK ? 16 * T_::B_STEP : T_::B_STEP;  // code bytes per step
  constexpr uint32_t B_PIECE = PK ? 1024 : 16;                   // between a lane's pieces
  constexpr uint32_t S_KS = PK ? 128 : 8;                         // scale bytes per step
  const int n = nsteps;

  // State of the tile whose K loop runs next: its coordinates, the row
  // count, the per-row scale (kept in a register until its epilogue) and the
  // load addresses.  Every address is a wave-uniform base plus one 32-bit
  // per-lane offset, so the loads use the scalar-base + 32-bit-offset form.
  int t_mt = 0, t_nt = 0, t_e = 0, t_nvalid = 0, t_mvalid = 0;
  float t_scale = 0.f;
  float t_ws[S == kW8A8 ? NSUB : 1];  // W8A8 weight scales of the K loop's tile
  int nrow[NSUB];
  const uint8_t* __restrict__ Bexp = B;
  const uint8_t* __restrict__ Sexp = reinterpret_cast<const uint8_t*>(g.b_scale);
  uint32_t boff[NSUB], soff[NSUB], aoff[NCH];
  // Bit offset of this lane's scale field in its aligned 32-bit word: the
  // field sits at byte 2*lane (streaming layout) or 2*lq (canonical) of a
  // 4-byte aligned run.
  const uint32_t sshift = ((PK ? lane : lq) & 1) * 16;

  auto load_b = [&](BFrag<S>(&bf)[NSUB], int ks) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < NSUB; s++) {
      const uint32_t o = boff[s] + (uint32_t)ks * B_KS;
      if constexpr (S == kW4A8 && !PK) {
        // Canonical W4A8: MFMA j's 8 codes of the lane are the 4 bytes at
        // 16j (+ 4 lq, in boff) of the row's step bytes.
#pragma unroll
        for (int j = 0; j < 4; j++)
          bf[s].q[0][j] = *reinterpret_cast<const uint32_t*>(Bexp + (uint32_t)(o + 16 * j));
      } else {
#pragma unroll
        for (int i = 0; i < T_::B_FRAG / 16; i++)
          bf[s].q[i] = *reinterpret_cast<const u32x4*>(Bexp + (uint32_t)(o + B_PIECE * i));
      }
      if constexpr (S == kW4A8) {
        // The four fp16 group scales of the lane's column for this step, 8
        // contiguous bytes in both layouts.
        typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 v =
            *reinterpret_cast<const u32x2*>(Sexp + (uint32_t)(soff[s] + ks * S_KS));
        bf[s].sc = v.x;
        bf[s].sc2 = v.y;
      } else if constexpr (S == kW4A16 || S == kA8W4) {
        // The lane's two scale bytes as part of the aligned 32-bit word that
        // holds them (a 16-bit load is zero-extended in the loop, which made
        // every fourth step wait for all loads in flight).
        bf[s].sc = *reinterpret_cast<const uint32_t*>(
            Sexp + ((uint32_t)(soff[s] + ks * S_KS) & ~3u));
      } else {
        bf[s].sc = 0;
      }
    }
  };
  auto load_a = [&](u32x4(&ar)[NCH], int ks) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NCH; i++)
      ar[i] = *reinterpret_cast<const u32x4*>(A + (uint32_t)(aoff[i] + ks * T_::A_STEP));
  };
  // Chunk i of this thread lands at LDS row (tid/CPR + i*kThreads/CPR).
  // (Skipping the rows of unused 16-row groups here was measured slower:
  // the branches cost more registers than the LDS writes they save.)
  auto store_a = [&](const u32x4(&ar)[NCH], int stage) __attribute__((always_inline)) {
    uint8_t* dst = sA(stage) + lds_w;
#pragma unroll
    for (int i = 0; i < NCH; i++) {
      if (NCH * kThreads == BM * CPR || tid + i * kThreads < BM * CPR)
        *reinterpret_cast<u32x4*>(dst + i * (kThreads / CPR) * PITCH) = ar[i];
    }
  };

  u32x4 ar[NCH];
  // The weight ring: RING register sets, loads RING-1 steps ahead.
  static_assert(RING == 4 || RING == 6 || RING == 8, "ring of 4, 6 or 8 steps");
  BFrag<S> bq[RING][NSUB];

  // Set-up of tile w, in four parts.  setup_rows: row ids into sRow[bf],
  // the row count, the weight offsets (no global loads).  setup_aoff: the
  // activation offsets.  meta_loads: the per-row scale of tile w and the
  // metadata of the tile after it.  setup_loads: the activation rows of
  // step 0 and the weights of steps 0 to RING-2.
  auto setup_rows = [&](int u, int bf) __attribute__((always_inline)) {
    decode(u, t_mt, t_nt);
    if (tid == kThreads - 1) sExpert[bf] = next_expert;
    int valid_here = 0;
    if (tid < BM) {
      const int ri = next_ri;
      sRow[bf][tid] = ri;
      valid_here = ri >= 0;
    }
    t_nvalid = __syncthreads_count(valid_here);
    t_mvalid = (t_nvalid + 15) >> 4;
    t_e = sExpert[bf];
    // Weight rows of this wave's sub-tiles, as 32-bit offsets from the
    // expert's base (one expert's weights are far below 4 GiB).
#pragma unroll
    for (int s = 0; s < NSUB; s++) {
      if (STAGE == 1) {
        const int base = t_nt * COLS + wave * HALF * 16 + lr;
        nrow[s] = s < HALF ? base + s * 16 : g.I + base + (s - HALF) * 16;
      } else {
        nrow[s] = t_nt * COLS + wave * NSUB * 16 + s * 16 + lr;
      }
    }
    Bexp = B + (size_t)t_e * g.N * kbytes;
    Sexp = reinterpret_cast<const uint8_t*>(g.b_scale) + (size_t)t_e * g.N * (K / 32) * SB;
    // Canonical layout: lane (lq, lr) reads row nrow's bytes [lq*B_FRAG,
    // (lq+1)*B_FRAG) of each step and the two scale bytes of that run.
    // Streaming layout (qmoe_prepack): the 16 rows x step bytes of a
    // sub-tile are one contiguous block in which the same bytes sit at
    // i*1024 + lane*16, and the step's scales are 128 contiguous bytes.
#pragma unroll
    for (int s = 0; s < NSUB; s++) {
      if constexpr (PK) {
        const uint32_t g16 = (uint32_t)(nrow[s] - lr);  // first row of the 16-row group
        boff[s] = g16 * (uint32_t)kbytes + lane * 16;
        // w4a8: 16 rows x 8 bytes per step, row lr's at 8 lr
        soff[s] = g16 * (uint32_t)(K / 32) * SB + (S == kW4A8 ? lr * 8 : lane * 2);
      } else {
        boff[s] = (uint32_t)nrow[s] * (uint32_t)kbytes + lq * (S == kW4A8 ? 4 : T_::B_FRAG);
        soff[s] = (uint32_t)nrow[s] * (uint32_t)(K / 32) * SB + (S == kW4A8 ? 0 : lq * 2);
      }
    }
  };
  // Activation chunks of this thread: fixed rows per tile.  Rows past the
  // tile's last real row read that row again (their results are dropped), so
  // every load is in bounds without a branch.
  auto setup_aoff = [&](int bf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NCH; i++) {
      const int row = min(tid / CPR + i * (kThreads / CPR), t_nvalid - 1), col = tid % CPR;
      const uint32_t rbase = STAGE == 1
                                 ? (uint32_t)sRow[bf][row] * (uint32_t)(g.H * T_::A_ELEM)
                                 : (uint32_t)(t_mt * BM + row) * (uint32_t)(g.I * T_::A_ELEM);
      aoff[i] = rbase + col * 16;
    }
  };
  auto meta_loads = [&](int u, int bf) __attribute__((always_inline)) {
    // Per-row scale of the epilogue (token scale in stage 1, the
    // requantized h scale in stage 2); the row id is read back from sRow.
    if constexpr (S != kW4A16) {
      if (tid < BM) {
        const int ri = sRow[bf][tid];
        t_scale = ri >= 0 ? g.a_scale[STAGE == 1 ? ri : (size_t)t_mt * BM + tid] : 0.f;
      }
    }
    fetch_meta(u + 1);
  };
  auto setup_loads = [&]() __attribute__((always_inline)) {
    load_a(ar, 0);
#pragma unroll
    for (int u = 0; u < RING - 1; u++) load_b(bq[u], min(u, n - 1));
  };

  Acc acc[MSUB][NSUB];
  int mvalid = 0;  // 16-row groups with a real row in the tile of the K loop

    // Activation fragments are read from LDS one 16-row group ahead of the
    // MFMAs that use them; the scheduling fences keep the compiler from
    // hoisting every group's reads (which would need ~8x the registers).
    auto read_frag = [&](u32x4(&af)[NF], int stage, int m) __attribute__((always_inline)) {
      const uint8_t* src = sA(stage) + (m * 16 + lr) * PITCH;
      if constexpr (S == kW4A8) {
        // MFMA j's 8 bytes: K [32j + 8 lq, +8) of the row; pieces 2f and
        // 2f + 1 share af[f].
        typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int f = 0; f < NF; f++) {
          const u32x2 p0 = *reinterpret_cast<const u32x2*>(src + 64 * f + 8 * lq);
          const u32x2 p1 = *reinterpret_cast<const u32x2*>(src + 64 * f + 32 + 8 * lq);
          af[f] = u32x4{p0.x, p0.y, p1.x, p1.y};
        }
      } else {
#pragma unroll
        for (int f = 0; f < NF; f++)
          af[f] = *reinterpret_cast<const u32x4*>(src + a_frag_offset<S, PK>(lq, f));
      }
    };
    // With FRAG2 the reads run one group ahead (two fragment buffers);
    // otherwise each group's reads directly precede its MFMAs and the other
    // wave on the SIMD covers the LDS latency (the 4-wave a8w4 128-row tile
    // has no registers left for the second buffer).  In tiles of 64 rows or
    // more the read ahead is unconditional (a group past the tile's rows
    // reads rows it never uses): were it skipped on some path, the counter
    // wait in front of the next group's MFMAs would have to assume the skip
    // and wait for every read in flight, the next group's too (measured:
    // stage 1 of the skewed W4A16 prefill 4% faster).  Shorter tiles, most
    // often one 16-row group full, keep the check: the unused reads cost
    // more there.
    constexpr bool FRAG2 = !(S == kA8W4 && BM >= 128 && (WAVES == 4 || STAGE == 2));
    auto compute = [&](int stage, const BFrag<S>(&bcr)[NSUB]) __attribute__((always_inline)) {
      BReady<S> bc[NSUB];
#pragma unroll
      for (int s = 0; s < NSUB; s++) bc[s] = prepare_b<S, PK>(bcr[s], sshift);
      u32x4 fa[NF], fb[NF];
      if constexpr (FRAG2) read_frag(fa, stage, 0);
#pragma unroll
      for (int m = 0; m < MSUB; m++) {
        if (m < mvalid) {
          if constexpr (FRAG2) {
            if (m + 1 < MSUB && (BM >= 64 || m + 1 < mvalid))
              read_frag((m & 1) ? fa : fb, stage, m + 1);
#pragma unroll
            for (int s = 0; s < NSUB; s++) mfma_step<S>(acc[m][s], (m & 1) ? fb : fa, bc[s]);
          } else {
            read_frag(fa, stage, m);
#pragma unroll
            for (int s = 0; s < NSUB; s++) mfma_step<S>(acc[m][s], fa, bc[s]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };

  // K loop.  Step s computes from LDS slot s%2 and weight register set
  // s%RING.  A step first writes the activation rows of step s+1 (loaded one
  // step earlier) to the other LDS slot, then issues the activation loads of
  // step s+2 and the weight loads of step s+RING-1 and runs the MFMAs of
  // step s; one barrier ends the step.  Load counters complete in order, so
  // issuing the activations first lets the wait for them skip the younger
  // weight loads.  The weight loads go in front of the MFMAs (LB false), or,
  // with LB (tall tiles full of rows), behind them: every wave of the block
  // issues its loads right after the barrier, and in front of a long run of
  // MFMAs they stalled each wave's issue until the CU's memory pipeline had
  // taken the block's 68 KiB of requests (a8w4 at 4096 tokens, timestamps
  // per phase: 920 of ~4000 clocks per step); behind the MFMAs that drain
  // overlaps them (stage 1 0.513 -> 0.492 ms), at the cost of issuing the
  // weights a little later, which short tiles cannot afford.  Loads past the
  // last step re-read the last step (cache hits): every step has the same
  // shape and the compiler's counter waits stay exact.
  auto step = [&](int s, const BFrag<S>(&bc)[NSUB], BFrag<S>(&bl)[NSUB])
      __attribute__((always_inline)) {
    store_a(ar, (s + 1) & 1);
    load_a(ar, min(s + 2, n - 1));
    if constexpr (LB) {
      if (s < n) compute(s & 1, bc);
      load_b(bl, min(s + RING - 1, n - 1));
    } else {
      load_b(bl, min(s + RING - 1, n - 1));
      if (s < n) compute(s & 1, bc);
    }
    __syncthreads();
  };
  // RING steps from s0 (a multiple of RING): step s0+u computes from ring
  // slot u and loads into the slot freed by the step before.
  auto group = [&](int s0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < RING; u++) step(s0 + u, bq[u], bq[(u + RING - 1) % RING]);
  };

  // The resident stage 2 that follows on the stream claims its work items
  // from per-XCD counters; they start from zero here (per-lane stores).
  if (STAGE == 1 && g.queue != nullptr && blockIdx.x == 0 && tid < 8) g.queue[tid] = 0;

  int wi = 0;  // the block's item counter
  if (!valid(0)) return;
  fetch_meta(wi);
  decode_meta();
  int buf = 0;
  setup_rows(wi, buf);
  setup_aoff(buf);
  meta_loads(wi, buf);
  setup_loads();
  bool first = true;
  while (true) {
    // The previous tile's output stores are still in flight.  On gfx9 stores
    // and loads share one counter, and pending stores would turn every wait
    // of the pipelined loop into a full drain; drain them here, where the
    // wait for this tile's first loads has to happen anyway.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    decode_meta();
    // W8A8: the per-channel weight scales of this tile's columns, loaded
    // before any of its K loop's loads, so that the epilogue's wait for them
    // does not wait for the next tile's loads already in flight.
    if constexpr (S == kW8A8) {
#pragma unroll
      for (int s = 0; s < NSUB; s++)
        t_ws[s] = reinterpret_cast<const float*>(g.b_scale)[(size_t)t_e * g.N + nrow[s]];
    }
    mvalid = t_mvalid;
#pragma unroll
    for (int m = 0; m < MSUB; m++)
#pragma unroll
      for (int s = 0; s < NSUB; s++) acc[m][s] = Acc{0, 0, 0, 0};
    if (!XT || first) {
      store_a(ar, 0);
      load_a(ar, min(1, n - 1));
      __syncthreads();
    }
    first = false;
    const int wn = wi + 1;
    const bool more = valid(wn);  // the same for the whole block

    // This tile's epilogue state (taken before the next tile's set-up).
    int mt, nt, e, nvalid, enrow[NSUB];
    float row_scale;
    const int ebuf = buf;
    auto keep_epilogue_state = [&]() __attribute__((always_inline)) {
      mt = t_mt, nt = t_nt, e = t_e, nvalid = t_nvalid;
      row_scale = t_scale;
#pragma unroll
      for (int s = 0; s < NSUB; s++) enrow[s] = nrow[s];
    };
    if constexpr (XT) {
      // n % RING == 0.  The last RING steps are written out: the loads that
      // would run past step n-1 fetch the next tile's activations of steps
      // 0-1 and weights of steps 0 to RING-2 instead (the current tile's last
      // step again when there is no next tile), into the slots and registers
      // that tile's step 0 expects.  Its row set-up runs before the first of
      // those weight loads, its activation offsets before the first of those
      // activation loads; neither has global loads of its own: a load issued
      // on only some paths would make every later counter wait of the loop a
      // conservative one.
      for (int s = 0; s < n - RING; s += RING) group(s);
      step(n - RING, bq[0], bq[RING - 1]);
#pragma unroll
      for (int u = 1; u < RING; u++) {
        const int s = n - RING + u;
        store_a(ar, (s + 1) & 1);
        if (u == RING - 2 && more) setup_aoff(buf ^ 1);
        load_a(ar, s + 2 < n ? s + 2 : (more ? s + 2 - n : n - 1));
        if (u == 1) {
          keep_epilogue_state();
          if (more) setup_rows(wn, buf ^ 1);
        }
        if constexpr (LB) {
          compute(s & 1, bq[u]);
          load_b(bq[u - 1], more ? u - 1 : n - 1);
        } else {
          load_b(bq[u - 1], more ? u - 1 : n - 1);
          compute(s & 1, bq[u]);
        }
        __syncthreads();
      }
    } else {
      for (int s = 0; s < n; s += RING) group(s);
      // The next tile's set-up and first loads run before this tile's
      // epilogue, so that those loads are in flight while the epilogue
      // computes and stores (issued after its stores they would queue
      // behind them).
      keep_epilogue_state();
      if (more) {
        setup_rows(wn, buf ^ 1);
        setup_aoff(buf ^ 1);
        meta_loads(wn, buf ^ 1);
        setup_loads();
      }
    }

    // ------------------------------------------------------------ epilogue
    // Phase 1: registers -> LDS tile (row = tile row, column = the block's
    // output column), after every wave is done with the activation ring.
    if (S != kW4A16 && tid < BM) sScale[tid] = row_scale;
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MSUB; m++) {
      if (m < mvalid) {
        // This lane's four rows m*16 + lq*4 + r: their ids and scales in
        // one 16-byte LDS read each.
        const int4 rid = *reinterpret_cast<const int4*>(&sRow[ebuf][m * 16 + lq * 4]);
        float4 rsc = make_float4(1.f, 1.f, 1.f, 1.f);
        if constexpr (S != kW4A16) rsc = *reinterpret_cast<const float4*>(&sScale[m * 16 + lq * 4]);
        const int rids[4] = {rid.x, rid.y, rid.z, rid.w};
        const float rscs[4] = {rsc.x, rsc.y, rsc.z, rsc.w};
#pragma unroll
        for (int r = 0; r < 4; r++) {
          const int row = m * 16 + lq * 4 + r;
          const size_t orow = (size_t)mt * BM + row;
          uint8_t* trow = etile + row * EPITCH;
          if constexpr (STAGE == 1) {
            const int tok = rids[r];
#pragma unroll
            for (int s = 0; s < HALF; s++) {
              const int cl = wave * HALF * 16 + s * 16 + lr;  // h column inside the tile
              float gf, uf;
              if constexpr (S == kW8A8) {
                const float xs = rscs[r];
                gf = ((float)acc[m][s][r] * xs) * t_ws[s];
                uf = ((float)acc[m][s + HALF][r] * xs) * t_ws[s + HALF];
                if (g.dump != nullptr && tok >= 0) {
                  g.dump[orow * 2 * g.I + enrow[s]] = acc[m][s][r];
                  g.dump[orow * 2 * g.I + enrow[s + HALF]] = acc[m][s + HALF][r];
                }
              } else if constexpr (S == kA8W4 || S == kW4A8) {
                const float xs = rscs[r];
                gf = acc[m][s][r] * xs;
                uf = acc[m][s + HALF][r] * xs;
                if (S == kW4A8 && g.dump != nullptr && tok >= 0) {
                  g.dump[orow * 2 * g.I + enrow[s]] = __float_as_int(acc[m][s][r]);
                  g.dump[orow * 2 * g.I + enrow[s + HALF]] = __float_as_int(acc[m][s + HALF][r]);
                }
              } else {
                gf = acc[m][s][r];
                uf = acc[m][s + HALF][r];
              }
              const float h = tok >= 0 ? silu_mul<S>(gf, uf) : 0.f;
              if constexpr (S == kW4A16)
                *reinterpret_cast<__bf16*>(trow + cl * 2) = (__bf16)h;
              else
                *reinterpret_cast<float*>(trow + cl * 4) = h;
            }
          } else {
            const int pair = rids[r];
            const float rs = rscs[r];
#pragma unroll
            for (int s = 0; s < NSUB; s++) {
              const int cl = wave * NSUB * 16 + s * 16 + lr;  // output column inside the tile
              if constexpr (S == kW8A8) {
                const float ws2 = t_ws[s];
                *reinterpret_cast<float*>(trow + cl * 4) = ((float)acc[m][s][r] * rs) * ws2;
                if (g.dump != nullptr && pair >= 0) g.dump[orow * g.H + enrow[s]] = acc[m][s][r];
              } else if constexpr (S == kA8W4 || S == kW4A8) {
                *reinterpret_cast<__bf16*>(trow + cl * 2) = (__bf16)(acc[m][s][r] * rs);
                if (S == kW4A8 && g.dump != nullptr && pair >= 0)
                  g.dump[orow * g.H + enrow[s]] = __float_as_int(acc[m][s][r]);
              } else {
                *reinterpret_cast<__bf16*>(trow + cl * 2) = (__bf16)acc[m][s][r];
              }
            }
          }
        }
      }
    }
    __syncthreads();
    // Phase 2: LDS tile -> global, 16 bytes per lane along each output row;
    // stage 1 of the requantized schemes also reduces each row's |h| max.
    {
      constexpr int CPRO = COLS * OUT_ES / 16;  // 16-byte chunks per output row
      constexpr int RPP = kThreads / CPRO;      // rows per pass
      static_assert(CPRO <= 64 && kThreads % CPRO == 0, "row chunks must fit a wave");
      const int prow = tid / CPRO, chunk = tid % CPRO;
      uint8_t* __restrict__ O = reinterpret_cast<uint8_t*>(g.out);
      for (int row0 = 0; row0 < mvalid * 16; row0 += RPP) {
        const int row = row0 + prow;
        const bool ok = row < nvalid;
        const u32x4 v = *reinterpret_cast<const u32x4*>(etile + (row < BM ? row : 0) * EPITCH +
                                                          chunk * 16);
        if constexpr (STAGE == 1) {
          if (ok)
            __builtin_nontemporal_store(
                v, reinterpret_cast<u32x4*>(O + ((size_t)mt * BM + row) * g.I * OUT_ES +
                                            (size_t)nt * COLS * OUT_ES + chunk * 16));
          if constexpr (S != kW4A16) {
            float a = fmaxf(fmaxf(fabsf(__uint_as_float(v.x)), fabsf(__uint_as_float(v.y))),
                            fmaxf(fabsf(__uint_as_float(v.z)), fabsf(__uint_as_float(v.w))));
            a = group_max<CPRO>(a);
            if (ok && chunk == CPRO - 1) g.row_pmax[((size_t)mt * BM + row) * g.ntiles_n + nt] = a;
          }
        } else {
          if (ok)
            __builtin_nontemporal_store(
                v, reinterpret_cast<u32x4*>(O + (size_t)sRow[ebuf][row] * g.H * OUT_ES +
                                            (size_t)nt * COLS * OUT_ES + chunk * 16));
        }
      }
    }
    if (!more) break;
    if constexpr (XT) meta_loads(wn, buf ^ 1);
    wi = wn;
    buf ^= 1;
    __syncthreads();  // the epilogue is done with the LDS tile before the next store_a
  }
}

template <int S, int STAGE, int BM, bool PK, int NSUB, int WAVES, bool XT, int RING,
          bool LB = false>
hipError_t launch_xt(const GemmArgs& g, hipStream_t s) {
  // Resident blocks per CU, queried once per kernel (a function-local
  // static: its initialisation is thread-safe).
  static const int blocks_per_cu = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, moe_gemm_kernel<S, STAGE, BM, PK, NSUB, WAVES, XT, RING, LB>, WAVES * 64, 0) !=
            hipSuccess ||
        n < 1)
      n = 1;
    return n;
  }();
  int nblk = device_cu_count() * blocks_per_cu;
  nblk = nblk < 8 ? 8 : (nblk / 8) * 8;
  hipLaunchKernelGGL((moe_gemm_kernel<S, STAGE, BM, PK, NSUB, WAVES, XT, RING, LB>), dim3(nblk),
                     dim3(WAVES * 64), 0, s, g);
  return hipGetLastError();
}

// Tiles of up to 32 rows (16 for a8w4, whose larger steps leave no
// registers for it at 32) stream few weight bytes per step, so their weight
// ring is eight steps long (seven steps of loads in flight) when the K loop
// has a multiple of eight steps; four otherwise.  Stage 1 runs the
// cross-tile pipeline whenever its K loop has a multiple of the ring's
// steps.
template <int S, int STAGE, int BM, bool PK, int NSUB, int WAVES>
hipError_t launch_one(const GemmArgs& g, int ring, int late_b, hipStream_t s) {
  const int nsteps = g.K / Tr<S>::BK;
  // The cross-tile pipeline: stage 1 of every scheme; stage 2 here runs
  // only for w4a16 and for long intermediates of the one-byte schemes
  // (otherwise the LDS-resident kernel takes it), where it stays off.
  constexpr bool XT2 = STAGE == 1 || S == kW4A16;
  if constexpr (BM <= (S == kA8W4 ? 16 : 32)) {
    if (nsteps % 8 == 0 && ring != 4)
      return launch_xt<S, STAGE, BM, PK, NSUB, WAVES, XT2, 8>(g, s);
  }
  if constexpr (BM == 128 && WAVES == 8) {
    // Weight loads behind the MFMAs when the tiles are mostly full (48 or
    // more rows per expert on average): measured 4-5% faster for a8w4 at
    // 4096 and 8192 tokens and the skewed W4A16 prefill, 1.6% slower at 1024
    // tokens (20 rows per expert).
    // (late_b: 1 forces this order, 0 the other one, -1 the rule.)
    const bool late = late_b >= 0 ? late_b == 1 : (long)g.P >= 48L * g.E;
    if (nsteps >= 4 && nsteps % 4 == 0 && late)
      return launch_xt<S, STAGE, BM, PK, NSUB, WAVES, XT2, 4, true>(g, s);
  }
  if (nsteps >= 4 && nsteps % 4 == 0)
    return launch_xt<S, STAGE, BM, PK, NSUB, WAVES, XT2, 4>(g, s);
  // w4a16 stage 2 with K = 768 (six steps): the whole K loop is one ring.
  if constexpr (STAGE == 2 && S == kW4A16 && BM <= 64) {
    if (nsteps == 6) return launch_xt<S, STAGE, BM, PK, NSUB, WAVES, true, 6>(g, s);
  }
  return launch_xt<S, STAGE, BM, PK, NSUB, WAVES, false, 4>(g, s);
}

template <int S, int STAGE, bool PK>
hipError_t launch_bm(int block_m, int nsub, int waves, int ring, int late_b, const GemmArgs& g,
                     hipStream_t s) {
#ifdef QMOE_ENABLE_WIDE
  if (nsub == 4 && waves == 4) {
    switch (block_m) {
      case 64: return launch_one<S, STAGE, 64, PK, 4, 4>(g, ring, late_b, s);
      case 128: return launch_one<S, STAGE, 128, PK, 4, 4>(g, ring, late_b, s);
      default: return hipErrorInvalidValue;
    }
  }
#endif
  if (nsub != 2) return hipErrorInvalidValue;
  if (waves == 8) {
    switch (block_m) {
      case 64: return launch_one<S, STAGE, 64, PK, 2, 8>(g, ring, late_b, s);
      case 128: return launch_one<S, STAGE, 128, PK, 2, 8>(g, ring, late_b, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (waves != 4) return hipErrorInvalidValue;
  switch (block_m) {
    case 16: return launch_one<S, STAGE, 16, PK, 2, 4>(g, ring, late_b, s);
    case 32: return launch_one<S, STAGE, 32, PK, 2, 4>(g, ring, late_b, s);
    case 64: return launch_one<S, STAGE, 64, PK, 2, 4>(g, ring, late_b, s);
    case 128: return launch_one<S, STAGE, 128, PK, 2, 4>(g, ring, late_b, s);
    default: return hipErrorInvalidValue;
  }
}

template <int S, int STAGE>
hipError_t launch_layout(bool packed, int block_m, int nsub, int waves, int ring, int late_b,
                         const GemmArgs& g, hipStream_t s) {
  return packed ? launch_bm<S, STAGE, true>(block_m, nsub, waves, ring, late_b, g, s)
                : launch_bm<S, STAGE, false>(block_m, nsub, waves, ring, late_b, g, s);
}

}  // namespace

hipError_t launch_gemm(int scheme, int stage, int block_m, bool packed, int nsub, int waves,
                       int ring, int late_b, const GemmArgs& g, hipStream_t s) {
  switch (scheme * 2 + (stage - 1)) {
    case 0: return launch_layout<kW4A16, 1>(packed, block_m, nsub, waves, ring, late_b, g, s);
    case 1: return launch_layout<kW4A16, 2>(packed, block_m, nsub, waves, ring, late_b, g, s);
    case 2: return launch_layout<kW8A8, 1>(packed, block_m, nsub, waves, ring, late_b, g, s);
    case 3: return launch_layout<kW8A8, 2>(packed, block_m, nsub, waves, ring, late_b, g, s);
    case 4: return launch_layout<kA8W4, 1>(packed, block_m, nsub, waves, ring, late_b, g, s);
    case 5: return launch_layout<kA8W4, 2>(packed, block_m, nsub, waves, ring, late_b, g, s);
    case 6: return launch_layout<kW4A8, 1>(packed, block_m, nsub, waves, ring, late_b, g, s);
    case 7: return launch_layout<kW4A8, 2>(packed, block_m, nsub, waves, ring, late_b, g, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qmoe
