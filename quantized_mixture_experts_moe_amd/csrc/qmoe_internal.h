// Internal declarations shared by the HIP sources of libqmoe (not installed).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmoe {

// Tile geometry of the grouped GEMMs (both stages).  A block is `waves`
// waves of 64 threads; every wave owns `nsub` 16-column weight sub-tiles and
// all BM rows of the tile, so a block covers waves*nsub*16 weight rows, and
// the gathered activation rows it stages in LDS feed all of them.
//  - 4 waves, nsub 2: two blocks share a CU (two waves per SIMD), so one
//    block's loads, epilogue and tile set-up overlap the other's MFMAs;
//  - 8 waves, nsub 2: one block per CU (two waves per SIMD); each staged
//    activation row feeds twice the weight rows, which halves the
//    activation traffic from L2 per weight byte;
//  - 4 waves, nsub 4 (wide): one block per CU, accumulators in AGPRs.
constexpr int kStages = 2;  // LDS slots of the activation ring
// h columns per stage-1 tile (gate and up sub-tiles pair up), output
// columns per stage-2 tile.
constexpr int stage_cols(int stage, int nsub, int waves) {
  return stage == 1 ? waves * nsub * 8 : waves * nsub * 16;
}
constexpr int kMinStage1Cols = stage_cols(1, 2, 4);  // sizes the per-row |h| max table

struct GemmArgs {
  int T, H, I, E, k, P;  // P = T*k pairs
  int N, K;              // this stage's GEMM N (weight rows) and K
  int ntiles_n;          // column tiles per row tile
  const int32_t* sorted_pair_ids;
  const int32_t* tile_expert;
  const int32_t* num_padded;
  const void* a;         // stage 1: x [T,H]; stage 2: h (quantized) [cap, I]
  const float* a_scale;  // stage 1: x_scale [T]; stage 2: h_scale [cap]
  const void* b;         // weight codes [E, N, K(/2)]
  const void* b_scale;   // weight scales
  void* out;             // stage 1: h (bf16 or f32) [cap, I]; stage 2: y_pairs [P, H]
  float* row_pmax;       // stage 1 (w8a8/a8w4): |h| max per row and column tile, written;
                         // resident stage 2: read, to quantize h while copying it
  int pmax_stride;       // column tiles of stage 1 (row pitch of row_pmax)
  int32_t* dump;         // w8a8 debug accumulators or nullptr
  int schedule;          // work order: 0 strided items, 1 runs of row tiles, 2 row tiles
                         // dealt to the XCDs
  int32_t* queue;        // stage 1: zeroes queue[0..7] (block 0); resident stage 2: the
                         // XCDs' work-item counters (nullptr: static split)
};

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                        hipStream_t s);
hipError_t launch_align(const int32_t* ids, int T, int k, int E, int block_m, int32_t* sorted,
                        int32_t* tile_expert, int32_t* offsets, int32_t* num_padded,
                        int32_t* chunk_counts, int32_t* chunk_flags, int32_t* totals,
                        int32_t* flags, int cap, hipStream_t s);
// ring: 0 = the depth the kernel picks (8 steps for tiles of up to 32 rows,
// 16 for a8w4, when the K loop has a multiple of 8 steps; else 4), 4 = four.
// late_b (128-row tiles of 8 waves): 1 = a step's weight loads behind its
// MFMAs, 0 = in front of them, -1 = by the rule (behind at 48 or more pairs
// per expert).
hipError_t launch_gemm(int scheme, int stage, int block_m, bool packed, int nsub, int waves,
                       int ring, int late_b, const GemmArgs& g, hipStream_t s);
// Stage 2 with the tile's activation rows resident in LDS (gemm_s2.hip):
// available for the one-byte-activation schemes with I <= 1024; its column
// passes are stage2_resident_cols() wide and a work item covers `passes`
// of them (ntiles_n must be a multiple of passes).  It reads stage 1's fp32
// h (g.a) and per-column-tile |h| maxima (g.row_pmax, g.pmax_stride) and
// quantizes each row as it copies it into LDS (no separate requant pass).
bool stage2_resident_ok(int scheme, int I);
int stage2_resident_cols();
int stage2_resident_max_passes(int scheme);  // bound on passes per work item
// half_tiles: each block_m-row tile is taken as two work items of
// block_m / 2 rows (an empty second half is skipped).
hipError_t launch_stage2_resident(int scheme, int block_m, bool half_tiles, bool packed,
                                  const GemmArgs& g, int passes, hipStream_t s);
hipError_t launch_prepack(int scheme, int E, int N, int K, const void* codes, const void* scales,
                          void* codes_out, void* scales_out, hipStream_t s);
hipError_t launch_requant(int scheme, const int32_t* sorted, const int32_t* num_padded,
                          int P, int I, int ntiles_n, int cap, const float* h32,
                          const float* pmax, uint8_t* hq, float* hs, hipStream_t s);
hipError_t launch_combine(const void* y, int y_f32, const float* w, int T, int k, int H,
                          uint16_t* out_bf16, float* out_f32, hipStream_t s);

size_t align_chunk_count(int T);
// Routing + grouping of up to route_align_fused_max_tokens() tokens in one
// launch of one block (align.hip).
int route_align_fused_max_tokens();
hipError_t launch_route_align(const float* logits, int T, int E, int k, int block_m,
                              int32_t* ids, float* w, int32_t* sorted, int32_t* tile_expert,
                              int32_t* offsets, int32_t* num_padded, int32_t* flags, int cap,
                              hipStream_t s);
int device_cu_count();

// The whole layer for up to decode_max_tokens() tokens in one launch
// (decode.hip).  Workspace byte offsets; the first counter_bytes hold the
// counters, which must be zero before the first call (every completed call
// leaves them zero).
struct DecodeWs {
  size_t flags, route_cnt, slot_flag, slot_rec, s1cnt, ready, ccnt, counter_bytes;
  size_t h32, pmax, hq, y, total;  // h32 and pmax: quantized schemes; hq: W4A16
};
int decode_max_tokens();
DecodeWs decode_ws_layout(int scheme, int H, int I, int E, int k);
// ring: weight + activation prefetch depth of a unit's K loop (4 or 6);
// chunks: 32-column chunks per stage-2 unit (1, 2, 4 or 8, with H / 32 a
// multiple of 4 * chunks).
int decode_stage2_chunks(int T, int H, int E, int k);
hipError_t launch_decode(int scheme, bool packed, int ring, int chunks, int T, int H, int I,
                         int E, int k,
                         const float* logits, const void* x, const float* x_scale,
                         const void* w13, const void* w13_scale, const void* w2,
                         const void* w2_scale, int32_t* topk_ids, float* topk_w, void* y,
                         uint16_t* out_bf16, float* out_f32, void* ws, uint64_t spin_ticks,
                         hipStream_t s);

}  // namespace qmoe
