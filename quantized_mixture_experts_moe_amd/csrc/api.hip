// Host side of the C ABI declared in include/qmoe.h: argument validation,
// workspace layout and kernel dispatch.  Nothing here allocates device
// memory or synchronises, except qmoe_check_flags.
#include <hip/hip_runtime.h>

#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "qmoe.h"
#include "qmoe_internal.h"

namespace qmoe {

static thread_local int g_last_hip_error = 0;

static qmoe_status hip_status(hipError_t e) {
  if (e == hipSuccess) return QMOE_OK;
  g_last_hip_error = (int)e;
  return QMOE_ERR_HIP;
}

int device_cu_count() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n < 1)
      n = 1;
    cached[dev] = n;
  }
  return cached[dev];
}

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Pairs up to which the resident stage 2 quantizes h itself (see
// grouped_ffn_impl).
constexpr int kFuseRequantPairs = 12288;
static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
static bool valid_block_m(int bm) { return bm == 16 || bm == 32 || bm == 64 || bm == 128; }

// Layout of qmoe_align's workspace: flag word, per-chunk flags, counts.
struct AlignWs {
  size_t flags, chunk_flags, counts, totals, total;
};
static AlignWs align_ws_layout(int T, int E) {
  AlignWs w;
  const size_t nch = align_chunk_count(T);
  w.flags = 0;
  w.chunk_flags = 256;
  w.counts = align_up(w.chunk_flags + nch * 4, 256);
  w.totals = align_up(w.counts + nch * (size_t)E * 4, 256);
  w.total = align_up(w.totals + (size_t)E * 4, 256);
  return w;
}

// Layout of qmoe_grouped_ffn's workspace.
struct FfnWs {
  size_t h, hq, hs, pmax, acc1, acc2, queue, total;
};
static FfnWs ffn_ws_layout(const qmoe_ffn_desc& d) {
  const size_t cap = qmoe_align_capacity(d.T, d.k, d.E, d.block_m);
  const size_t I = d.I, H = d.H;
  FfnWs w{};
  size_t off = 0;
  w.h = off;
  off = align_up(off + cap * I * (d.scheme == QMOE_W4A16_G32 ? 2 : 4), 256);
  if (d.scheme != QMOE_W4A16_G32) {
    // The quantized h and its row scales are materialized unless the
    // resident stage 2 quantizes while it copies.
    if (!stage2_resident_ok(d.scheme, d.I) || (size_t)d.T * d.k > (size_t)kFuseRequantPairs) {
      w.hq = off;
      off = align_up(off + cap * I, 256);
      w.hs = off;
      off = align_up(off + cap * 4, 256);
    }
    w.pmax = off;
    off = align_up(off + cap * (I / kMinStage1Cols) * 4, 256);
  }
  if ((d.scheme == QMOE_W8A8_PERCHAN || d.scheme == QMOE_W4A8_G32) &&
      (d.flags & QMOE_FLAG_DUMP_ACC)) {
    w.acc1 = off;
    off = align_up(off + cap * 2 * I * 4, 256);
    w.acc2 = off;
    off = align_up(off + cap * H * 4, 256);
  }
  // The resident stage 2's per-XCD work-item counters (stage 1 zeroes them).
  w.queue = off;
  off = align_up(off + 8 * 4, 256);
  w.total = off;
  return w;
}

// ---------------------------------------------------------------------------
// Tile configuration of one grouped-FFN call.  Every choice here changes
// only how the work is split (tile heights, blocks, prefetch depth, column
// passes), never the order or precision of a sum, so all give the same bits.
struct TileCfg {
  int s1_waves;   // stage-1 block: 4 or 8 waves (8 needs block_m >= 64); 0 = rule
  int s1_ring;    // stage-1 weight prefetch ring: 0 = kernel's pick, 4 = four steps
  int s1_runs;    // stage-1 schedule: -1 = rule, 0 = strided items, 1 = runs of row tiles,
                  // 2 = row tiles dealt to the XCDs (also stage 2's, row-major kernel)
  int s2_waves;   // row-major stage 2 (W4A16, W4A8, I > 1024): as s1_waves
  int s2_passes;  // resident stage 2: column passes per work item; 0 = rule
  int s2_half;    // resident stage 2: -1 = rule, 0 = whole tiles, 1 = half tiles
  // Stage-1 weight loads behind the MFMAs: -1 = rule, 0 = in front, 1 =
  // behind (tile-table rows leave it out: the rule).
  int s1_late = -1;
  // Resident stage 2: work items claimed from per-XCD counters (-1 = rule:
  // with half tiles, 1 = on, 0 = the static split).
  int s2_queue = -1;
};
constexpr TileCfg kRuleCfg = {0, 0, -1, 0, 0, -1, -1};

struct TileRow {
  int scheme, H, I, E, k, t_max, block_m;
  TileCfg cfg;
};
static const TileRow kTileTable[] = {
#include "tile_table.inc"
    {-1, 0, 0, 0, 0, 0, 0, kRuleCfg}};  // end marker

static const TileRow* table_row(int scheme, int T, int H, int I, int E, int k) {
  for (const TileRow* r = kTileTable; r->scheme >= 0; r++)
    if (r->scheme == scheme && r->H == H && r->I == I && r->E == E && r->k == k && T <= r->t_max)
      return r;
  return nullptr;
}

// Tile height by rule, from the mean rows per expert (pairs / E), where the
// table has no row: up to 12 rows per expert 16; up to 40, 64 (one or two
// tiles per expert); up to 96, 128 (one tile per expert, weights read once);
// above, 64 (a second 128-row tile would be mostly padding), except a8w4
// with an intermediate of 1024 or more above 128 rows, where 128-row tiles
// taken in runs (an expert's second tile reads its weights from the
// memory-side cache) measured faster.
static int rule_block_m(int scheme, int T, int I, int E, int k) {
  const double mean_rows = (double)T * k / E;
  if (mean_rows <= 12) return 16;
  if (mean_rows <= 40) return 64;
  if (mean_rows <= 96) return 128;
  if (scheme == QMOE_A8W4_MXFP4 && mean_rows > 128 && I >= 1024) return 128;
  return 64;
}

// QMOE_TILE="s1w=8,s1r=4,s1runs=1,s2w=4,s2p=8,s2h=0" overrides fields of the
// configuration (for tile sweeps).  Returns false on a malformed string.
static bool parse_tile_env(TileCfg& c) {
  const char* e = getenv("QMOE_TILE");
  if (e == nullptr || *e == 0) return true;
  const char* p = e;
  while (*p) {
    const char* eq = strchr(p, '=');
    if (eq == nullptr) return false;
    const std::string key(p, eq - p);
    char* end = nullptr;
    const long v = strtol(eq + 1, &end, 10);
    if (end == eq + 1) return false;
    if (key == "s1w") c.s1_waves = (int)v;
    else if (key == "s1r") c.s1_ring = (int)v;
    else if (key == "s1runs") c.s1_runs = (int)v;
    else if (key == "s2w") c.s2_waves = (int)v;
    else if (key == "s2p") c.s2_passes = (int)v;
    else if (key == "s2h") c.s2_half = (int)v;
    else if (key == "s1lb") c.s1_late = (int)v;
    else if (key == "s2q") c.s2_queue = (int)v;
    else return false;
    p = end;
    if (*p == ',') p++;
    else if (*p != 0) return false;
  }
  return true;
}

// Block shape of the grouped GEMMs: sub-tiles per wave and waves per block.
// 8-wave blocks (one per CU) halve the activation traffic per weight byte;
// measured on the 128-row tiles they win for stage 1 of the 4-bit-weight
// schemes and stage 2 of W8A8, and the 4-wave blocks (two per CU) win the
// other stage.  Smaller tiles keep 4-wave blocks.  The wide tiles (one
// 4-wave block per CU, AGPR accumulators) measured slower everywhere and are
// built only with QMOE_ENABLE_WIDE.
struct GemmShape {
  int nsub, waves;
};
static GemmShape choose_shape(int scheme, int stage, int block_m) {
#ifdef QMOE_ENABLE_WIDE
  if (block_m >= 64) return {4, 4};
#endif
  const int wide_stage = scheme == QMOE_W8A8_PERCHAN ? 2 : 1;
  if (block_m >= 128 && stage == wide_stage) return {2, 8};
  return {2, 4};
}

static qmoe_status check_desc(const qmoe_ffn_desc* d) {
  if (d == nullptr) return QMOE_ERR_INVALID_ARG;
  if (d->scheme < 0 || d->scheme > 3) return QMOE_ERR_INVALID_ARG;
  if (d->T < 0 || d->H <= 0 || d->I <= 0 || d->E <= 0 || d->k < 1 || d->k > d->E)
    return QMOE_ERR_INVALID_ARG;
  if (d->H % 32 != 0 || d->I % 32 != 0) return QMOE_ERR_INVALID_ARG;
  if (!valid_block_m(d->block_m)) return QMOE_ERR_INVALID_ARG;
  if ((long long)d->T * d->k > (1ll << 30)) return QMOE_ERR_INVALID_ARG;
  if (d->flags & ~(QMOE_FLAG_DUMP_ACC | QMOE_FLAG_PREPACKED)) return QMOE_ERR_INVALID_ARG;
  if (d->E > 1024) return QMOE_ERR_UNSUPPORTED;
  if (d->H % 256 != 0) return QMOE_ERR_UNSUPPORTED;
  if (d->I % (d->scheme == QMOE_A8W4_MXFP4 ? 256 : 128) != 0) return QMOE_ERR_UNSUPPORTED;
  return QMOE_OK;
}

// Descriptor check of qmoe_decode (block_m is not used).
static qmoe_status check_decode_desc(const qmoe_ffn_desc* d) {
  if (d == nullptr) return QMOE_ERR_INVALID_ARG;
  if (d->scheme < 0 || d->scheme > 3) return QMOE_ERR_INVALID_ARG;
  if (d->T < 0 || d->H <= 0 || d->I <= 0 || d->E <= 0 || d->k < 1 || d->k > d->E || d->k > 16)
    return QMOE_ERR_INVALID_ARG;
  if (d->H % 32 != 0 || d->I % 32 != 0) return QMOE_ERR_INVALID_ARG;
  if (d->flags & ~QMOE_FLAG_PREPACKED) return QMOE_ERR_INVALID_ARG;
  if (d->T > decode_max_tokens() || d->E > 1024) return QMOE_ERR_UNSUPPORTED;
  if (d->scheme != QMOE_W4A16_G32 && d->I > QMOE_DECODE_MAX_INTER) return QMOE_ERR_UNSUPPORTED;
  if (d->H % 256 != 0) return QMOE_ERR_UNSUPPORTED;
  if (d->I % (d->scheme == QMOE_A8W4_MXFP4 ? 256 : 128) != 0) return QMOE_ERR_UNSUPPORTED;
  // One expert's W13 or W2 codes are addressed with 32-bit byte offsets.
  const uint64_t wrow = d->scheme == QMOE_W8A8_PERCHAN ? 2 : 1;  // weight bytes per 2 elements
  if ((uint64_t)2 * d->I * d->H * wrow / 2 >= (1ull << 32)) return QMOE_ERR_UNSUPPORTED;
  return QMOE_OK;
}

// A wait inside the decode kernel gives up after 100 ms of the device's
// constant-rate clock.
static uint64_t decode_spin_ticks() {
  static std::mutex mu;
  static uint64_t cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == 0) {
    int khz = 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess ||
        khz < 1)
      khz = 100000;
    cached[dev] = (uint64_t)khz * 100;
  }
  return cached[dev];
}

// Prefetch depth of the decode kernel's K loops: QMOE_DECODE_RING (4 or 6)
// or 4.  0 for an invalid value.  (QMOE_DECODE_G, read in qmoe_decode,
// overrides the stage-2 chunks per unit for measurements.)
static int decode_ring() {
  const char* e = getenv("QMOE_DECODE_RING");
  if (e == nullptr || *e == 0) return 4;
  if (strcmp(e, "4") == 0) return 4;
  if (strcmp(e, "6") == 0) return 6;
  return 0;
}

}  // namespace qmoe

using namespace qmoe;

extern "C" {

int qmoe_abi_version(void) { return QMOE_ABI_VERSION; }

const char* qmoe_status_str(qmoe_status s) {
  switch (s) {
    case QMOE_OK: return "ok";
    case QMOE_ERR_INVALID_ARG: return "invalid argument";
    case QMOE_ERR_UNSUPPORTED: return "unsupported shape or scheme";
    case QMOE_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int qmoe_last_hip_error(void) { return g_last_hip_error; }

qmoe_status qmoe_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* topk_ids,
                       float* topk_w, void* stream) {
  if (T < 0 || E < 1 || k < 1 || k > E || k > 16) return QMOE_ERR_INVALID_ARG;
  if (E > 1024) return QMOE_ERR_UNSUPPORTED;
  if (T == 0) return QMOE_OK;
  if (!logits || !topk_ids || !topk_w) return QMOE_ERR_INVALID_ARG;
  return hip_status(launch_route(logits, T, E, k, topk_ids, topk_w, (hipStream_t)stream));
}

int32_t qmoe_default_block_m(int32_t scheme, int32_t T, int32_t H, int32_t I, int32_t E,
                             int32_t k) {
  if (scheme < 0 || scheme > 3 || T < 0 || H <= 0 || I <= 0 || E < 1 || k < 1 || k > E)
    return 0;
  if (const TileRow* row = table_row(scheme, T, H, I, E, k)) return row->block_m;
  return rule_block_m(scheme, T, I, E, k);
}

size_t qmoe_align_capacity(int32_t T, int32_t k, int32_t E, int32_t block_m) {
  if (T < 0 || k < 1 || E < 1 || !valid_block_m(block_m)) return 0;
  const size_t P = (size_t)T * k;
  const size_t cap = P + std::min<size_t>((size_t)E, P) * (size_t)(block_m - 1);
  return align_up(std::max<size_t>(cap, 1), (size_t)block_m);
}

size_t qmoe_align_workspace(int32_t T, int32_t k, int32_t E) {
  (void)k;
  if (T < 0 || E < 1) return 0;
  return align_ws_layout(T, E).total;
}

qmoe_status qmoe_align(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E, int32_t block_m,
                       int32_t* sorted_pair_ids, int32_t* tile_expert, int32_t* expert_offsets,
                       int32_t* num_padded, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || k < 1 || E < 1 || k > E || !valid_block_m(block_m)) return QMOE_ERR_INVALID_ARG;
  if ((long long)T * k > (1ll << 30)) return QMOE_ERR_INVALID_ARG;
  if (E > 1024) return QMOE_ERR_UNSUPPORTED;
  if ((T > 0 && !topk_ids) || !sorted_pair_ids || !tile_expert || !expert_offsets ||
      !num_padded || !ws)
    return QMOE_ERR_INVALID_ARG;
  const AlignWs lay = align_ws_layout(T, E);
  if (ws_bytes < lay.total || !aligned(ws, 256)) return QMOE_ERR_INVALID_ARG;
  const int cap = (int)qmoe_align_capacity(T, k, E, block_m);
  uint8_t* w = reinterpret_cast<uint8_t*>(ws);
  return hip_status(launch_align(topk_ids, T, k, E, block_m, sorted_pair_ids, tile_expert,
                                 expert_offsets, num_padded,
                                 reinterpret_cast<int32_t*>(w + lay.counts),
                                 reinterpret_cast<int32_t*>(w + lay.chunk_flags),
                                 reinterpret_cast<int32_t*>(w + lay.totals),
                                 reinterpret_cast<int32_t*>(w + lay.flags), cap,
                                 (hipStream_t)stream));
}

qmoe_status qmoe_route_align(const float* logits, int32_t T, int32_t E, int32_t k,
                             int32_t block_m, int32_t* topk_ids, float* topk_w,
                             int32_t* sorted_pair_ids, int32_t* tile_expert,
                             int32_t* expert_offsets, int32_t* num_padded, void* ws,
                             size_t ws_bytes, void* stream) {
  if (T < 0 || E < 1 || k < 1 || k > E || k > 16 || !valid_block_m(block_m))
    return QMOE_ERR_INVALID_ARG;
  if (E > 1024) return QMOE_ERR_UNSUPPORTED;
  if ((T > 0 && (!logits || !topk_ids || !topk_w)) || !sorted_pair_ids || !tile_expert ||
      !expert_offsets || !num_padded || !ws)
    return QMOE_ERR_INVALID_ARG;
  const AlignWs lay = align_ws_layout(T, E);
  if (ws_bytes < lay.total || !aligned(ws, 256)) return QMOE_ERR_INVALID_ARG;
  const int cap = (int)qmoe_align_capacity(T, k, E, block_m);
  uint8_t* w = reinterpret_cast<uint8_t*>(ws);
  hipStream_t s = (hipStream_t)stream;
  if (T >= 1 && T <= route_align_fused_max_tokens())
    return hip_status(launch_route_align(logits, T, E, k, block_m, topk_ids, topk_w,
                                         sorted_pair_ids, tile_expert, expert_offsets,
                                         num_padded, reinterpret_cast<int32_t*>(w + lay.flags),
                                         cap, s));
  if (T > 0) {
    const hipError_t e = launch_route(logits, T, E, k, topk_ids, topk_w, s);
    if (e != hipSuccess) return hip_status(e);
  }
  return hip_status(launch_align(topk_ids, T, k, E, block_m, sorted_pair_ids, tile_expert,
                                 expert_offsets, num_padded,
                                 reinterpret_cast<int32_t*>(w + lay.counts),
                                 reinterpret_cast<int32_t*>(w + lay.chunk_flags),
                                 reinterpret_cast<int32_t*>(w + lay.totals),
                                 reinterpret_cast<int32_t*>(w + lay.flags), cap, s));
}

// ---------------------------------------------------------------------------
// qmoe_align_noalloc: qmoe_align with its workspace in a file-scope device
// array instead of a caller buffer, for callers that cannot allocate.
//
// The array is statically sized (QMOE_ALIGN_NOALLOC_MAX_BYTES); every GPU the
// library runs on holds its own copy until the process ends.  In host code
// `scratch` only names the symbol: its device address on the current device
// comes from hipGetSymbolAddress, taken once per device on the first call
// there and cached below; only that address is ever passed to a kernel.
static __device__ __align__(256) uint8_t scratch[QMOE_ALIGN_NOALLOC_MAX_BYTES];

static hipError_t scratch_ptr(uint8_t** out) {
  static std::mutex mu;
  static uint8_t* cached[64] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    cached[dev] = reinterpret_cast<uint8_t*>(p);
  }
  *out = cached[dev];
  return hipSuccess;
}

qmoe_status qmoe_align_noalloc(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E,
                               int32_t block_m, int32_t* sorted_pair_ids,
                               int32_t* tile_expert, int32_t* expert_offsets,
                               int32_t* num_padded, int32_t* flags, void* stream) {
  if (T < 0 || k < 1 || E < 1 || k > E || !valid_block_m(block_m)) return QMOE_ERR_INVALID_ARG;
  if ((long long)T * k > (1ll << 30)) return QMOE_ERR_INVALID_ARG;
  if (E > 1024) return QMOE_ERR_UNSUPPORTED;
  if ((T > 0 && !topk_ids) || !sorted_pair_ids || !tile_expert || !expert_offsets ||
      !num_padded)
    return QMOE_ERR_INVALID_ARG;
  const AlignWs lay = align_ws_layout(T, E);
  if (lay.total > (size_t)QMOE_ALIGN_NOALLOC_MAX_BYTES) return QMOE_ERR_UNSUPPORTED;
  uint8_t* w = nullptr;
  hipError_t e = scratch_ptr(&w);
  if (e != hipSuccess) return hip_status(e);
  // Every region of the workspace is written before it is read within one
  // call (counts and chunk flags by the count kernel, totals and the flag
  // word by the scan or place kernel), so nothing is cleared first.
  const int cap = (int)qmoe_align_capacity(T, k, E, block_m);
  int32_t* fl = flags ? flags : reinterpret_cast<int32_t*>(w + lay.flags);
  return hip_status(launch_align(topk_ids, T, k, E, block_m, sorted_pair_ids, tile_expert,
                                 expert_offsets, num_padded,
                                 reinterpret_cast<int32_t*>(w + lay.counts),
                                 reinterpret_cast<int32_t*>(w + lay.chunk_flags),
                                 reinterpret_cast<int32_t*>(w + lay.totals), fl, cap,
                                 (hipStream_t)stream));
}

qmoe_status qmoe_check_flags(const void* align_ws, int32_t* flags_out, void* stream) {
  if (!align_ws || !flags_out) return QMOE_ERR_INVALID_ARG;
  int32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, align_ws, sizeof(int32_t), hipMemcpyDeviceToHost,
                                (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e);
  *flags_out = v;
  return QMOE_OK;
}

size_t qmoe_grouped_ffn_workspace(const qmoe_ffn_desc* d) {
  if (check_desc(d) != QMOE_OK) return 0;
  return ffn_ws_layout(*d).total;
}

qmoe_status qmoe_grouped_ffn_debug_offsets(const qmoe_ffn_desc* d, size_t* acc1_off,
                                           size_t* acc2_off) {
  const qmoe_status st = check_desc(d);
  if (st != QMOE_OK) return st;
  if ((d->scheme != QMOE_W8A8_PERCHAN && d->scheme != QMOE_W4A8_G32) ||
      !(d->flags & QMOE_FLAG_DUMP_ACC) || !acc1_off ||
      !acc2_off)
    return QMOE_ERR_INVALID_ARG;
  const FfnWs lay = ffn_ws_layout(*d);
  *acc1_off = lay.acc1;
  *acc2_off = lay.acc2;
  return QMOE_OK;
}

static qmoe_status grouped_ffn_impl(const qmoe_ffn_desc* d, const void* x, const float* x_scale,
                                    const qmoe_weights* w, const int32_t* sorted_pair_ids,
                                    const int32_t* tile_expert, const int32_t* num_padded,
                                    void* y_pairs, void* ws, size_t ws_bytes,
                                    void* const* events, void* stream) {
  const qmoe_status st = check_desc(d);
  if (st != QMOE_OK) return st;
  if (d->T == 0) return QMOE_OK;
  const bool quant_act = d->scheme != QMOE_W4A16_G32;
  if (!x || !w || !w->w13 || !w->w13_scale || !w->w2 || !w->w2_scale || !sorted_pair_ids ||
      !tile_expert || !num_padded || !y_pairs || !ws || (quant_act && !x_scale))
    return QMOE_ERR_INVALID_ARG;
  const size_t scale_align = d->scheme == QMOE_W4A8_G32 ? 8 : 4;  // w4a8: 8-byte scale loads
  if (!aligned(x, 16) || !aligned(w->w13, 16) || !aligned(w->w2, 16) || !aligned(ws, 256) ||
      !aligned(y_pairs, 16) || !aligned(w->w13_scale, scale_align) ||
      !aligned(w->w2_scale, scale_align))
    return QMOE_ERR_INVALID_ARG;
  const FfnWs lay = ffn_ws_layout(*d);
  if (ws_bytes < lay.total) return QMOE_ERR_INVALID_ARG;
  // The GEMM kernels address activation rows and one expert's weights with
  // 32-bit byte offsets: x [T, H], the stage-2 activations [cap, I] and each
  // expert's W13 / W2 codes must stay below 4 GiB.
  {
    const uint64_t lim = 1ull << 32;
    const uint64_t ab = quant_act ? 1 : 2;  // bytes per activation element
    const uint64_t capu = qmoe_align_capacity(d->T, d->k, d->E, d->block_m);
    const uint64_t wrow = d->scheme == QMOE_W8A8_PERCHAN ? 2 : 1;  // weight bytes per 2 elements
    if ((uint64_t)d->T * d->H * ab >= lim || capu * d->I * ab >= lim ||
        (uint64_t)2 * d->I * d->H * wrow / 2 >= lim || (uint64_t)d->H * d->I * wrow / 2 >= lim)
      return QMOE_ERR_UNSUPPORTED;
  }
  uint8_t* wsb = reinterpret_cast<uint8_t*>(ws);
  const bool dump = (d->scheme == QMOE_W8A8_PERCHAN || d->scheme == QMOE_W4A8_G32) &&
                    (d->flags & QMOE_FLAG_DUMP_ACC);
  const int cap = (int)qmoe_align_capacity(d->T, d->k, d->E, d->block_m);
  hipStream_t s = (hipStream_t)stream;

  GemmArgs g1{};
  g1.T = d->T;
  g1.H = d->H;
  g1.I = d->I;
  g1.E = d->E;
  g1.k = d->k;
  g1.P = d->T * d->k;
  g1.sorted_pair_ids = sorted_pair_ids;
  g1.tile_expert = tile_expert;
  g1.num_padded = num_padded;
  GemmArgs g2 = g1;

  // Tile configuration: the table's row for this shape and token bucket
  // when its block_m is the caller's, else the rules; QMOE_TILE overrides.
  TileCfg cfg = kRuleCfg;
  if (const TileRow* row = table_row(d->scheme, d->T, d->H, d->I, d->E, d->k))
    if (row->block_m == d->block_m) cfg = row->cfg;
  if (!parse_tile_env(cfg)) return QMOE_ERR_INVALID_ARG;
  const bool resident = stage2_resident_ok(d->scheme, d->I);
  GemmShape gs1 = choose_shape(d->scheme, 1, d->block_m);
  GemmShape gs2 = choose_shape(d->scheme, 2, d->block_m);
  auto waves_ok = [&](int w) { return w == 0 || w == 4 || (w == 8 && d->block_m >= 64); };
  if (!waves_ok(cfg.s1_waves) || !waves_ok(cfg.s2_waves) ||
      (cfg.s1_ring != 0 && cfg.s1_ring != 4) || cfg.s1_runs < -1 || cfg.s1_runs > 2 ||
      cfg.s2_half < -1 || cfg.s2_half > 1 || cfg.s2_passes < 0 || cfg.s1_late < -1 ||
      cfg.s1_late > 1 || cfg.s2_queue < -1 || cfg.s2_queue > 1 ||
      (cfg.s2_half == 1 && (!resident || d->block_m < 32)) ||
      (cfg.s2_passes > 0 && !resident) || (cfg.s2_waves != 0 && resident))
    return QMOE_ERR_INVALID_ARG;
  if (cfg.s1_waves) gs1.waves = cfg.s1_waves;
  if (cfg.s2_waves) gs2.waves = cfg.s2_waves;

  g1.N = 2 * d->I;
  g1.K = d->H;
  g1.ntiles_n = d->I / stage_cols(1, gs1.nsub, gs1.waves);
  g1.a = x;
  g1.a_scale = x_scale;
  g1.b = w->w13;
  g1.b_scale = w->w13_scale;
  g1.out = wsb + lay.h;
  g1.row_pmax = quant_act ? reinterpret_cast<float*>(wsb + lay.pmax) : nullptr;
  g1.dump = dump ? reinterpret_cast<int32_t*>(wsb + lay.acc1) : nullptr;
  // a8w4 with 128-row tiles and more pairs than one tile per expert: the
  // stage-1 blocks take runs of consecutive row tiles (an expert's second
  // tile then reads its weights from the memory-side cache); measured
  // neutral or slower for the other schemes and tile heights.
  // W4A16 and W4A8 tiles of 64 rows or more over 256 experts or more: row
  // tiles dealt to the XCDs, so that each XCD gets the same mix of full and
  // partial tiles (skewed 8192-token prefill over 512 experts: W4A16 step
  // 2.76 -> 2.65 ms, W4A8 4.50 -> 4.23 ms; the 2048-token W4A8 step over 128
  // experts, whose tiles are all about full, 2-3% slower with it, and the
  // a8w4 8192-token step, which takes runs, 4.5% slower).
  g1.schedule = (d->scheme == QMOE_A8W4_MXFP4 && d->block_m == 128 &&
                 (long)d->T * d->k > (long)d->E * d->block_m)
                    ? 1
                : ((d->scheme == QMOE_W4A16_G32 || d->scheme == QMOE_W4A8_G32) &&
                   d->block_m >= 64 && d->E >= 256)
                    ? 2
                    : 0;
  if (cfg.s1_runs >= 0) g1.schedule = cfg.s1_runs;
  // Stage-2 work split, settled (and checked) before anything is launched.
  // Where stage 1 takes runs of row tiles (several 128-row tiles per
  // expert), stage 2 takes each tile as two 64-row work items.
  const bool half_tiles =
      resident && (cfg.s2_half >= 0 ? cfg.s2_half == 1 : g1.schedule == 1 && d->block_m >= 32);
  int passes = 1;
  if (resident) {
    // Column passes per work item: as many as keep at least four items per
    // CU (by the capacity's tile count), so every item copies its rows to
    // LDS once for as many passes as possible.
    g2.ntiles_n = d->H / stage2_resident_cols();
    const long tiles = (long)cap / (half_tiles ? d->block_m / 2 : d->block_m);
    for (int p = g2.ntiles_n; p >= 1; p--) {
      if (g2.ntiles_n % p != 0 || p > stage2_resident_max_passes(d->scheme)) continue;
      passes = p;
      if (tiles * (g2.ntiles_n / p) >= 4L * device_cu_count()) break;
    }
    if (cfg.s2_passes > 0) {
      if (g2.ntiles_n % cfg.s2_passes != 0 ||
          cfg.s2_passes > stage2_resident_max_passes(d->scheme))
        return QMOE_ERR_INVALID_ARG;
      passes = cfg.s2_passes;
    }
  } else {
    g2.ntiles_n = d->H / stage_cols(2, gs2.nsub, gs2.waves);
  }

  // With half tiles the resident stage 2 balances its items through
  // per-XCD counters that stage 1 zeroes: at 8192 tokens of the a8w4 block
  // about a quarter of the half tiles hold no rows, and the static split
  // left blocks idle for a quarter of the kernel (stage 2 0.601 -> 0.481
  // ms).  With whole tiles the items cost about the same and the claim's
  // round trip at each item measured 1-4% slower.
  const bool use_queue = resident && (cfg.s2_queue >= 0 ? cfg.s2_queue == 1 : half_tiles);
  int32_t* const queue = use_queue ? reinterpret_cast<int32_t*>(wsb + lay.queue) : nullptr;
  g1.queue = queue;
  g2.queue = queue;

  auto mark = [&](int i) -> hipError_t {
    return events ? hipEventRecord((hipEvent_t)events[i], s) : hipSuccess;
  };
  hipError_t e = mark(0);
  const bool packed = (d->flags & QMOE_FLAG_PREPACKED) != 0;
  if (e == hipSuccess)
    e = launch_gemm(d->scheme, 1, d->block_m, packed, gs1.nsub, gs1.waves, cfg.s1_ring,
                    cfg.s1_late, g1, s);
  if (e == hipSuccess) e = mark(1);
  if (e != hipSuccess) return hip_status(e);

  // The resident stage 2 quantizes h itself while it copies each row tile
  // into LDS (one launch and one pass over h fewer) up to kFuseRequantPairs
  // pairs.  Beyond that its copy of fp32 rows, which no other block on the
  // CU overlaps, cost more than the separate pass (measured: 4096 tokens of
  // the a8w4 block, stage 2 334 -> 416 us against 54 us of requantization;
  // at 256 and 1024 tokens the fused form is 6-8 us faster).
  const bool fuse_requant = quant_act && resident && g1.P <= kFuseRequantPairs;
  if (quant_act && !fuse_requant) {
    e = launch_requant(d->scheme, sorted_pair_ids, num_padded, g1.P, d->I, g1.ntiles_n, cap,
                       reinterpret_cast<const float*>(wsb + lay.h),
                       reinterpret_cast<const float*>(wsb + lay.pmax), wsb + lay.hq,
                       reinterpret_cast<float*>(wsb + lay.hs), s);
    if (e != hipSuccess) return hip_status(e);
  }
  e = mark(2);
  if (e != hipSuccess) return hip_status(e);

  g2.schedule = g1.schedule == 2 ? 2 : 0;  // the resident stage 2 splits its own work
  g2.N = d->H;
  g2.K = d->I;
  if (fuse_requant) {
    // fp32 h and the per-column-tile maxima; quantized in the row copy.
    g2.a = wsb + lay.h;
    g2.a_scale = nullptr;
    g2.row_pmax = reinterpret_cast<float*>(wsb + lay.pmax);
    g2.pmax_stride = g1.ntiles_n;
  } else {
    g2.a = quant_act ? (const void*)(wsb + lay.hq) : (const void*)(wsb + lay.h);
    g2.a_scale = quant_act ? reinterpret_cast<const float*>(wsb + lay.hs) : nullptr;
    g2.row_pmax = nullptr;
    g2.pmax_stride = 0;
  }
  g2.b = w->w2;
  g2.b_scale = w->w2_scale;
  g2.out = y_pairs;
  g2.dump = dump ? reinterpret_cast<int32_t*>(wsb + lay.acc2) : nullptr;
  e = resident ? launch_stage2_resident(d->scheme, d->block_m, half_tiles, packed, g2, passes, s)
               : launch_gemm(d->scheme, 2, d->block_m, packed, gs2.nsub, gs2.waves, 0, -1, g2, s);
  if (e == hipSuccess) e = mark(3);
  return hip_status(e);
}

}  // extern "C" (reopened below)

extern "C" {

qmoe_status qmoe_grouped_ffn(const qmoe_ffn_desc* d, const void* x, const float* x_scale,
                             const qmoe_weights* w, const int32_t* sorted_pair_ids,
                             const int32_t* tile_expert, const int32_t* num_padded, void* y_pairs,
                             void* ws, size_t ws_bytes, void* stream) {
  return grouped_ffn_impl(d, x, x_scale, w, sorted_pair_ids, tile_expert, num_padded, y_pairs, ws,
                          ws_bytes, nullptr, stream);
}

qmoe_status qmoe_grouped_ffn_profiled(const qmoe_ffn_desc* d, const void* x,
                                      const float* x_scale, const qmoe_weights* w,
                                      const int32_t* sorted_pair_ids,
                                      const int32_t* tile_expert, const int32_t* num_padded,
                                      void* y_pairs, void* ws, size_t ws_bytes,
                                      void* const stage_events[4], void* stream) {
  if (!stage_events || !stage_events[0] || !stage_events[1] || !stage_events[2] ||
      !stage_events[3])
    return QMOE_ERR_INVALID_ARG;
  return grouped_ffn_impl(d, x, x_scale, w, sorted_pair_ids, tile_expert, num_padded, y_pairs, ws,
                          ws_bytes, stage_events, stream);
}

qmoe_status qmoe_prepack(int32_t scheme, int32_t E, int32_t N, int32_t K, const void* codes,
                         const void* scales, void* codes_out, void* scales_out, void* stream) {
  if (scheme < 0 || scheme > 3 || E < 1 || N < 1 || K < 1) return QMOE_ERR_INVALID_ARG;
  if (N % 16 != 0 || K % (scheme == QMOE_A8W4_MXFP4 ? 256 : 128) != 0) return QMOE_ERR_INVALID_ARG;
  if ((long long)E * N > (1ll << 31)) return QMOE_ERR_INVALID_ARG;
  if (!codes || !codes_out || !scales) return QMOE_ERR_INVALID_ARG;
  if (scheme != QMOE_W8A8_PERCHAN && !scales_out) return QMOE_ERR_INVALID_ARG;
  if (!aligned(codes, 16) || !aligned(codes_out, 16) || !aligned(scales, 4) ||
      (scales_out && !aligned(scales_out, 4)))
    return QMOE_ERR_INVALID_ARG;
  const size_t cb = (size_t)E * N * (scheme == QMOE_W8A8_PERCHAN ? K : K / 2);
  const size_t sbytes = scheme == QMOE_W8A8_PERCHAN
                            ? (size_t)E * N * 4
                            : (size_t)E * N * (K / 32) * (scheme == QMOE_A8W4_MXFP4 ? 1 : 2);
  auto overlap = [](const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
  };
  if (overlap(codes, cb, codes_out, cb) ||
      (scales_out && overlap(scales, sbytes, scales_out, sbytes)))
    return QMOE_ERR_INVALID_ARG;
  return hip_status(launch_prepack(scheme, E, N, K, codes, scales, codes_out, scales_out,
                                   (hipStream_t)stream));
}

qmoe_status qmoe_combine(const void* y_pairs, int32_t y_dtype, const float* topk_w, int32_t T,
                         int32_t k, int32_t H, uint16_t* out_bf16, float* out_f32, void* stream) {
  if (T < 0 || k < 1 || H <= 0 || H % 8 != 0) return QMOE_ERR_INVALID_ARG;
  if (y_dtype != QMOE_DT_BF16 && y_dtype != QMOE_DT_F32) return QMOE_ERR_INVALID_ARG;
  if (T == 0) return QMOE_OK;  // nothing to write (the outputs may be empty, null buffers)
  if (!out_bf16 && !out_f32) return QMOE_ERR_INVALID_ARG;
  if (!y_pairs || !topk_w) return QMOE_ERR_INVALID_ARG;
  if (!aligned(y_pairs, 16) || (out_bf16 && !aligned(out_bf16, 16)) ||
      (out_f32 && !aligned(out_f32, 16)))
    return QMOE_ERR_INVALID_ARG;
  return hip_status(launch_combine(y_pairs, y_dtype == QMOE_DT_F32, topk_w, T, k, H, out_bf16,
                                   out_f32, (hipStream_t)stream));
}

size_t qmoe_decode_workspace(const qmoe_ffn_desc* d) {
  if (check_decode_desc(d) != QMOE_OK) return 0;
  return decode_ws_layout(d->scheme, d->H, d->I, d->E, d->k).total;
}

qmoe_status qmoe_decode(const qmoe_ffn_desc* d, const float* logits, const void* x,
                        const float* x_scale, const qmoe_weights* w, int32_t* topk_ids,
                        float* topk_w, void* y_pairs, uint16_t* out_bf16, float* out_f32,
                        void* ws, size_t ws_bytes, void* stream) {
  const qmoe_status st = check_decode_desc(d);
  if (st != QMOE_OK) return st;
  if (d->T == 0) return QMOE_OK;
  const bool quant_act = d->scheme != QMOE_W4A16_G32;
  if (!logits || !x || !w || !w->w13 || !w->w13_scale || !w->w2 || !w->w2_scale || !topk_ids ||
      !topk_w || !ws || (quant_act && !x_scale) || (!out_bf16 && !out_f32))
    return QMOE_ERR_INVALID_ARG;
  const size_t scale_align = d->scheme == QMOE_W4A8_G32 ? 8 : 4;
  if (!aligned(x, 16) || !aligned(w->w13, 16) || !aligned(w->w2, 16) || !aligned(ws, 256) ||
      !aligned(w->w13_scale, scale_align) || !aligned(w->w2_scale, scale_align) ||
      (y_pairs && !aligned(y_pairs, 16)))
    return QMOE_ERR_INVALID_ARG;
  if (ws_bytes < decode_ws_layout(d->scheme, d->H, d->I, d->E, d->k).total)
    return QMOE_ERR_INVALID_ARG;
  const int ring = decode_ring();
  if (ring == 0) return QMOE_ERR_INVALID_ARG;
  int chunks = decode_stage2_chunks(d->T, d->H, d->E, d->k);
  if (const char* e = getenv("QMOE_DECODE_G"); e != nullptr && *e != 0) {
    chunks = atoi(e);
    if ((chunks != 1 && chunks != 2 && chunks != 4 && chunks != 8) ||
        (d->H / 32) % (4 * chunks) != 0)
      return QMOE_ERR_INVALID_ARG;
  }
  return hip_status(launch_decode(d->scheme, (d->flags & QMOE_FLAG_PREPACKED) != 0, ring,
                                  chunks, d->T,
                                  d->H, d->I, d->E, d->k, logits, x, x_scale, w->w13,
                                  w->w13_scale, w->w2, w->w2_scale, topk_ids, topk_w, y_pairs,
                                  out_bf16, out_f32, ws, decode_spin_ticks(),
                                  (hipStream_t)stream));
}

}  // extern "C"
