// The whole MoE layer for a small batch (up to 16 tokens) in one launch:
// routing, grouping, stage 1 with the fused silu(gate)*up epilogue, the
// scheme's per-row requantization of h, stage 2 and the fixed-order weighted
// combine.  In the decode regime every expert GEMM has a handful of rows and
// the step is bound by weight streaming and by the number of dependent
// launches (vLLM issue "Evaluate native IU4/IU8 WMMA for grouped-INT MoE
// prefill on gfx1151", section Problem; aiter PR 6090, section Changes:
// token bucket 1-256); here the dependencies are resolved inside the launch.
//
// Work units.  Every wave of the grid is one unit, numbered in launch order
// (workgroup b holds units 4b .. 4b+3):
//   [0, u0)                     route token u < T (one wave per token; u0 is
//                               T rounded up to whole workgroups);
//   then smax * c1 stage-1 units (slot j, 16 h columns c: the 16 gate and
//                               16 up weight rows of those columns, all K);
//   then smax * c2 stage-2 units (slot j, G chunks of 32 output columns,
//                               all K each; G = 4 where H / 32 allows).
// c1 and c2 are multiples of four, so the four units of a workgroup always
// belong to one slot and one stage.  (Numbering the units slot by slot, a
// slot's stage-2 units right behind its stage-1 units, measured slower: its
// stage-2 waves hold their wave slots while the slot's stage 1 runs.)  A slot is one of the experts the batch
// touches (ascending expert id); it holds the rows (pairs, ascending)
// routed to it, at most T <= 16 of them, so one 16-row MFMA tile covers
// every slot.  smax = min(E, T*k) bounds the number of slots; units of
// slots past the actual count end at once.
//
// Dependencies run only from a unit to units with smaller numbers:
//  - the last routing wave to finish (an arrival counter) groups the pairs
//    into slots and then publishes every slot's record (expert, rows),
//    which releases the slot's workgroups;
//  - stage-1 workgroups wait for their slot's record; the last stage-1 unit
//    of a slot to finish sets ready[j];
//  - stage-2 workgroups wait for the record, issue their weight loads, then
//    wait for ready[j] and (quantized schemes) requantize the slot's h rows
//    into their LDS;
//  - the last stage-2 unit to write its 32 columns of a token's k rows
//    (ccnt[t][c]) combines them.
// One wave per workgroup polls a flag (of its copy, see kCopies) and hands
// the result to the other three through LDS.  Workgroups are dispatched in
// index order, so the units a wave waits for have been dispatched before
// it: they run to completion whether or not the whole grid is resident, and
// no wait can wait for a unit that is not running.  Each wait is still
// bounded (spin_ticks of the constant-rate clock); a wait that runs out
// sets kDecodeTimeout in the flag word and carries on, so the launch always
// ends.
//
// Every counter returns to zero by the end of a call (each is reset by its
// last user), so a workspace zeroed once serves any number of calls ordered
// on one stream.
//
// Numerics are those of the grouped path, step for step: the same MFMA
// sequence per output (K steps ascending), the same epilogue recipes, the
// row scale from the row's |h| maximum and the correctly rounded quotient of
// quant_common.h, and the combine's slot-order fp32 sum; outputs equal the
// route -> align -> grouped FFN -> combine sequence bit for bit.
#include <algorithm>

#include "gemm_common.h"
#include "quant_common.h"
#include "route_common.h"

namespace qmoe {
namespace {

using namespace gk;

constexpr int kWaves = 4;        // waves per workgroup; each wave is its own unit
constexpr int kMaxTokens = 16;   // rows of one MFMA tile
constexpr int32_t kDecodeTimeout = 4;  // flag-word bit: a wait ran out of time
// Every flag that many workgroups wait for exists in kCopies copies; the
// workgroup b polls copy b % kCopies (one wave per workgroup polls), so that
// no single address takes the polls of the whole grid.
constexpr int kCopies = 8;

// Workgroups in [lo, hi) whose index is x modulo kCopies.
__host__ __device__ inline int count_mod(int lo, int hi, int x) {
  auto upto = [x](int v) { return v > x ? (v - x + kCopies - 1) / kCopies : 0; };
  return upto(hi) - upto(lo);
}

struct DecodeArgs {
  int T, H, I, E, k, P, smax, c1, c2;
  int G;   // 32-column chunks per stage-2 unit (c2 = H / (32 G) units per slot)
  int u0;  // first stage-1 unit (T rounded up to whole workgroups; 0 with local routing)
  int local_route;  // every workgroup routes the batch itself (T <= 2)
  const float* logits;
  const void* x;
  const float* x_scale;
  const void* w13;
  const void* w13_scale;
  const void* w2;
  const void* w2_scale;
  int32_t* topk_ids;
  float* topk_w;
  void* y;  // [P, H]: bf16, fp32 for W8A8
  uint16_t* out_bf16;
  float* out_f32;
  int32_t* flags;
  int32_t* route_cnt;    // [1]
  int32_t* slot_rec;     // [smax, 8]: the slot records (see group_pairs)
  int32_t* slot_flag;    // [kCopies, smax]: workgroups still to pass the record
  int32_t* s1cnt;        // [smax]: stage-1 units finished
  int32_t* ready;        // [kCopies, smax]: stage-2 workgroups still to pass, once h is
                         // quantized
  int32_t* ccnt;         // [T, c2]: stage-2 units finished per token and column group
  float* h32;            // [P, I]: fp32 h (requantized schemes)
  float* pmax;           // [P, c1]: |h| max per 16 columns
  void* hq;              // [P, I]: W4A16's bf16 h (the quantized schemes requantize
                         // h32 into each stage-2 workgroup's LDS)
  uint64_t spin_ticks;
};

__device__ inline int32_t atomic_add(int32_t* p, int32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void atomic_set(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Data passed between waves (the routing results, the slot tables, h, its
// codes and scales, y) is written and read with device-coherent accesses
// (relaxed atomics at agent scope: they bypass the caches that are private
// to an XCD), so no cache of the chip has to be written back or invalidated
// at a hand-over: a producer waits until its stores have completed and
// then sets the counter or flag; a consumer reads the data after it has
// seen the flag.  (Agent-scope fences instead write back and invalidate the
// whole L2 of the XCD at every hand-over, thousands per launch.)
template <class V>
__device__ inline void cstore(V* p, V v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class V>
__device__ inline V cload(const V* p) {
  return __hip_atomic_load(const_cast<V*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Every store of the wave issued so far has completed (and the compiler
// keeps memory accesses on their side of this point).
__device__ inline void release() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Memory accesses after this point stay after the flag read before it.
__device__ inline void acquire() { asm volatile("" ::: "memory"); }
// Orders this wave's LDS accesses across its lanes (LDS serves one wave's
// accesses in order; this only keeps the compiler from moving them).
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Lane 0 adds v; every lane gets the old value.
__device__ inline int32_t wave_add(int32_t* p, int32_t v) {
  int32_t old = 0;
  if ((threadIdx.x & 63) == 0) old = atomic_add(p, v);
  return __builtin_amdgcn_readfirstlane(old);
}

// Waits until *p is non-zero (bounded), then acquires.
__device__ inline void wait_set(const int32_t* p, const DecodeArgs& g) {
  const uint64_t t0 = wall_clock64();
  int nap = 1;
  while (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) {
    if (wall_clock64() - t0 > g.spin_ticks) {
      if ((threadIdx.x & 63) == 0)
        __hip_atomic_fetch_or(g.flags, kDecodeTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    // Back off: polls that reach memory compete with the weight streams.
    for (int q = 0; q < nap; q++) __builtin_amdgcn_s_sleep(2);
    nap = nap < 8 ? nap + 1 : 8;
  }
  acquire();
}

__device__ inline float wave_max(float a) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
  return a;
}

// ---------------------------------------------------------------- routing
// LDS of the grouping step (one wave of a workgroup at most runs it).
struct AlignLds {
  int32_t ids[2 * kMaxTokens * 16];  // pair ids, then each slot's expert
  uint32_t bits[32];
  int32_t pre[32];
  int32_t cnt[kMaxTokens * 16];
  uint8_t rows[kMaxTokens * 16 * kMaxTokens];  // [slot][row]: pair id (< 256)
  float wts[kWaves * 16];                      // routing weights (local routing)
};

// Groups the P = T*k pairs into slots: slot = rank of the pair's expert among
// the touched experts, row = rank of the pair among that expert's pairs
// (pair order).  One wave; P <= 256, E <= 1024.  The pairs' expert ids are
// in L.ids already when ids_ready (one token: its own routing), else they
// are read back from topk_ids.
//
// Slot record j (8 words, read by one wave of each of the slot's workgroups
// in one round trip after the slot's flag is set): word 0 = expert | rows
// << 16 (rows 0: no expert, the workgroups end at once); words 1-4 = the
// rows' pair ids, one byte each.  The flag (slot_flag, kCopies copies) holds
// the workgroups still to pass: those of the slot that poll the copy, when
// published; each decrements it, so it is zero again at the end of the
// call.
// First workgroup of slot j's stage-1 and stage-2 units.
__device__ inline int stage1_block(const DecodeArgs& g, int j) {
  return (g.u0 + j * g.c1) / kWaves;
}
__device__ inline int stage2_block(const DecodeArgs& g, int j) {
  return (g.u0 + g.smax * g.c1 + j * g.c2) / kWaves;
}

// The grouping in LDS (one wave): L.cnt[slot] = rows, L.rows[slot][row] =
// pair id, L.ids[P + slot] = expert; returns the number of slots.
__device__ int group_core(const DecodeArgs& g, AlignLds& L) {
  const int lane = threadIdx.x & 63;
  const int P = g.P, W = (g.E + 31) >> 5;
  if (lane < 32) L.bits[lane] = 0u;
  wave_lds_sync();
  for (int i = lane; i < P; i += 64) {
    const int e = L.ids[i];
    atomicOr(&L.bits[e >> 5], 1u << (e & 31));
  }
  wave_lds_sync();
  // Slot of the first touched expert of each 32-expert word.
  const int c = lane < W ? __popc(L.bits[lane]) : 0;
  int incl = c;
#pragma unroll
  for (int off = 1; off < 32; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if ((lane & 31) >= off) incl += y;
  }
  if (lane < 32) L.pre[lane] = incl - c;
  const int nact = __builtin_amdgcn_readlane(incl, 31);
  for (int s = lane; s < nact; s += 64) L.cnt[s] = 0;
  wave_lds_sync();
  for (int base = 0; base < P; base += 64) {
    const int i = base + lane;
    const int id = i < P ? L.ids[i] : -1;
    int before = 0, after = 0;
    for (int l = 0; l < 64; l++) {
      const int o = __builtin_amdgcn_readlane(id, l);
      if (o == id) {
        before += l < lane;
        after += l > lane;
      }
    }
    if (i < P) {
      const int w = id >> 5;
      const int slot = L.pre[w] + __popc(L.bits[w] & ((1u << (id & 31)) - 1u));
      const int rank = L.cnt[slot] + before;
      L.rows[slot * kMaxTokens + rank] = (uint8_t)i;
      if (rank == 0) L.ids[P + slot] = id;  // past the pairs: the slot's expert
      if (after == 0) L.cnt[slot] = rank + 1;
    }
    wave_lds_sync();
  }
  return nact;
}

// Record word w (0-4) of slot j (see group_pairs), from the LDS grouping.
__device__ inline uint32_t record_word(const DecodeArgs& g, const AlignLds& L, int nact, int j,
                                       int w) {
  if (j >= nact) return 0u;
  if (w == 0) return (uint32_t)L.ids[g.P + j] | ((uint32_t)L.cnt[j] << 16);
  const uint8_t* r = &L.rows[j * kMaxTokens + 4 * (w - 1)];
  return (uint32_t)r[0] | ((uint32_t)r[1] << 8) | ((uint32_t)r[2] << 16) | ((uint32_t)r[3] << 24);
}

__device__ void group_pairs(const DecodeArgs& g, AlignLds& L, bool ids_ready) {
  const int lane = threadIdx.x & 63;
  if (!ids_ready)
    for (int i = lane; i < g.P; i += 64) L.ids[i] = cload(&g.topk_ids[i]);
  wave_lds_sync();
  const int nact = group_core(g, L);
  // Words 0-4 of every record (rows 0 for the slots past nact).
  for (int idx = lane; idx < g.smax * 5; idx += 64) {
    const int j = idx / 5, w = idx - 5 * (idx / 5);
    cstore(reinterpret_cast<uint32_t*>(&g.slot_rec[j * 8 + w]), record_word(g, L, nact, j, w));
  }
  release();
  for (int idx = lane; idx < kCopies * g.smax; idx += 64) {
    const int x = idx / g.smax, j = idx - x * g.smax;
    const int b1 = stage1_block(g, j), b2 = stage2_block(g, j);
    const int n = count_mod(b1, b1 + g.c1 / kWaves, x) + count_mod(b2, b2 + g.c2 / kWaves, x);
    if (n > 0) atomic_set(&g.slot_flag[x * g.smax + j], n);
  }
}

__device__ inline void route_one(const DecodeArgs& g, int t, int* e, float* w) {
  const float* row = g.logits + (size_t)t * g.E;
  if (g.E <= 256)
    rt::route_token<4>(row, g.E, g.k, e, w);
  else if (g.E <= 512)
    rt::route_token<8>(row, g.E, g.k, e, w);
  else
    rt::route_token<16>(row, g.E, g.k, e, w);
}

// Local routing (T <= 2 <= kWaves): every workgroup routes the whole batch
// itself, wave t routing token t, and groups it in LDS; it keeps its own
// slot's record in s_rec and the routing weights in L.wts.  Workgroup 0
// also writes topk_ids and topk_w.  No unit waits for another's routing.
__device__ void route_local(const DecodeArgs& g, AlignLds& L, int j, uint32_t* s_rec) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (wave < g.T) {
    int e = 0;
    float w = 0.f;
    route_one(g, wave, &e, &w);
    if (lane < g.k) {
      L.ids[wave * g.k + lane] = e;
      L.wts[wave * g.k + lane] = w;
      if (blockIdx.x == 0) {
        g.topk_ids[wave * g.k + lane] = e;
        g.topk_w[wave * g.k + lane] = w;
      }
    }
  }
  __syncthreads();
  if (wave == 0) {
    const int nact = group_core(g, L);
    if (lane < 5) s_rec[lane] = record_word(g, L, nact, j, lane);
  }
  __syncthreads();
}

__device__ void route_unit(const DecodeArgs& g, int t, AlignLds& L) {
  const int lane = threadIdx.x & 63;
  int e = 0;
  float w = 0.f;
  route_one(g, t, &e, &w);
  if (lane < g.k) {
    cstore(&g.topk_ids[t * g.k + lane], e);
    cstore(&g.topk_w[t * g.k + lane], w);
  }
  if (g.T == 1) {
    // One token: its wave groups its own pairs (no arrival to count).
    if (lane < g.k) L.ids[lane] = e;
    wave_lds_sync();
    group_pairs(g, L, true);
    return;
  }
  release();
  if (wave_add(g.route_cnt, 1) != g.T - 1) return;
  // The last token routed: no other wave touches route_cnt in this call.
  if (lane == 0) atomic_set(g.route_cnt, 0);
  acquire();
  group_pairs(g, L, false);
}

// ------------------------------------------------------------ expert GEMMs
// One ring slot: a K step's weight fragments of the wave's two 16-row
// sub-tiles and its activation fragment.
template <int S>
struct Slot {
  BFrag<S> b[2];
  u32x4 a[Tr<S>::A_FRAG / 16];
};

// Where a unit's activation rows are read from: global memory written
// before the launch (x), global memory another wave wrote (device-coherent
// loads), or this workgroup's LDS.
enum ASrc { kFromGlobal, kFromCoherent, kFromLds };

// One K step of a unit: the loads of a ring slot and its MFMAs.  The
// weight loads of sub-tile s start at code byte boff[s] and scale byte
// soff[s] (K step 0); the activation loads at arow.
template <int S, bool PK, int SRC>
struct KStep {
  using T_ = Tr<S>;
  using Acc = typename T_::Acc;
  static constexpr int NF = T_::A_FRAG / 16;
  static constexpr uint32_t B_KS = PK ? 16 * T_::B_STEP : T_::B_STEP;
  static constexpr uint32_t B_PIECE = PK ? 1024 : 16;
  static constexpr uint32_t S_KS = PK ? 128 : 8;
  const uint8_t* __restrict__ B;
  const uint8_t* __restrict__ Sc;
  const uint8_t* __restrict__ arow;
  int lq;
  uint32_t sshift;

  __device__ KStep(const uint8_t* b, const uint8_t* sc, const uint8_t* a) : B(b), Sc(sc), arow(a) {
    const int lane = threadIdx.x & 63;
    lq = lane >> 4;
    sshift = ((PK ? lane : lq) & 1) * 16;
  }

  __device__ __attribute__((always_inline)) void load_b(Slot<S>& sl, const uint32_t (&boff)[2],
                                                       const uint32_t (&soff)[2], int ks) const {
#pragma unroll
    for (int s = 0; s < 2; s++) {
      const uint32_t o = boff[s] + (uint32_t)ks * B_KS;
      if constexpr (S == kW4A8 && !PK) {
#pragma unroll
        for (int j = 0; j < 4; j++)
          sl.b[s].q[0][j] = *reinterpret_cast<const uint32_t*>(B + (uint32_t)(o + 16 * j));
      } else {
#pragma unroll
        for (int i = 0; i < T_::B_FRAG / 16; i++)
          sl.b[s].q[i] = *reinterpret_cast<const u32x4*>(B + (uint32_t)(o + B_PIECE * i));
      }
      if constexpr (S == kW4A8) {
        typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 v = *reinterpret_cast<const u32x2*>(Sc + (uint32_t)(soff[s] + ks * S_KS));
        sl.b[s].sc = v.x;
        sl.b[s].sc2 = v.y;
      } else if constexpr (S == kW4A16 || S == kA8W4) {
        sl.b[s].sc = *reinterpret_cast<const uint32_t*>(Sc + ((uint32_t)(soff[s] + ks * S_KS) & ~3u));
      } else {
        sl.b[s].sc = 0;
      }
    }
  }
  __device__ __attribute__((always_inline)) void load_a(Slot<S>& sl, int ks) const {
    const uint8_t* src = arow + (uint32_t)ks * T_::A_STEP;
    if constexpr (SRC == kFromLds) {
      typedef __attribute__((address_space(3))) const uint8_t lds_u8;
      typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
      const lds_u8* ls = (const lds_u8*)src;
#pragma unroll
      for (int f = 0; f < NF; f++) {
        if constexpr (S == kW4A8) {
          const u32x2 p0 = *reinterpret_cast<const __attribute__((address_space(3))) u32x2*>(
              ls + 64 * f + 8 * lq);
          const u32x2 p1 = *reinterpret_cast<const __attribute__((address_space(3))) u32x2*>(
              ls + 64 * f + 32 + 8 * lq);
          sl.a[f] = u32x4{p0.x, p0.y, p1.x, p1.y};
        } else {
          sl.a[f] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
              ls + a_frag_offset<S, PK>(lq, f));
        }
      }
    } else if constexpr (SRC == kFromCoherent) {
      // Another wave wrote these rows: four device-coherent 32-bit loads
      // per 16 bytes (W4A8: two per 8-byte piece).
      auto w32 = [&](int off) __attribute__((always_inline)) {
        return cload(reinterpret_cast<const uint32_t*>(src + off));
      };
#pragma unroll
      for (int f = 0; f < NF; f++) {
        if constexpr (S == kW4A8) {
          const int o0 = 64 * f + 8 * lq, o1 = 64 * f + 32 + 8 * lq;
          sl.a[f] = u32x4{w32(o0), w32(o0 + 4), w32(o1), w32(o1 + 4)};
        } else {
          const int o = a_frag_offset<S, PK>(lq, f);
          sl.a[f] = u32x4{w32(o), w32(o + 4), w32(o + 8), w32(o + 12)};
        }
      }
    } else if constexpr (S == kW4A8) {
      typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
      for (int f = 0; f < NF; f++) {
        const u32x2 p0 = *reinterpret_cast<const u32x2*>(src + 64 * f + 8 * lq);
        const u32x2 p1 = *reinterpret_cast<const u32x2*>(src + 64 * f + 32 + 8 * lq);
        sl.a[f] = u32x4{p0.x, p0.y, p1.x, p1.y};
      }
    } else {
#pragma unroll
      for (int f = 0; f < NF; f++)
        sl.a[f] = *reinterpret_cast<const u32x4*>(src + a_frag_offset<S, PK>(lq, f));
    }
  }
  __device__ __attribute__((always_inline)) void compute(Acc (&acc)[2], const Slot<S>& sl) const {
#pragma unroll
    for (int s = 0; s < 2; s++) mfma_step<S>(acc[s], sl.a, prepare_b<S, PK>(sl.b[s], sshift));
  }
  // 24 wait states after the MFMAs wherever control may leave a run of
  // steps (a loop's back edge and exit, each step of a tail): the register
  // allocator copies the accumulators between register files at those
  // edges, and the compiler's wait-state count there measured short on
  // gfx950: a copy of the last accumulator register 8 wait states after
  // v_mfma_i32_16x16x64_i8 (ahead of the other three, which came at 9-11)
  // still held the previous step's sum.  Every other read of an MFMA result
  // in this kernel comes at least 11 wait states after it.
  __device__ static __attribute__((always_inline)) void pad() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
    __builtin_amdgcn_sched_barrier(0);
  }
};

// The K loop of one unit: acc[s] += rows (16, A) x weight rows of sub-tile s,
// K steps 0..n-1 in order.  The weight loads of the first R steps are issued
// before wait() returns; the activation loads after it.
template <int S, bool PK, int R, int SRC, class Wait>
__device__ inline void k_loop(const KStep<S, PK, SRC>& ks, const uint32_t (&boff)[2],
                              const uint32_t (&soff)[2], int n, typename Tr<S>::Acc (&acc)[2],
                              Wait wait) {
  Slot<S> ring[R];
  if (n >= R) {
    // Steady state: step s computes from ring[s % R], then loads step s + R
    // into it.  Every load of the main loop is unconditional, so the
    // compiler's counter waits stay exact; the tail (the last R to 2R-1
    // steps) loads only what is still needed.
#pragma unroll
    for (int u = 0; u < R; u++) ks.load_b(ring[u], boff, soff, u);
    wait();
#pragma unroll
    for (int u = 0; u < R; u++) ks.load_a(ring[u], u);
    int s0 = 0;
    for (; s0 + 2 * R <= n; s0 += R) {
#pragma unroll
      for (int u = 0; u < R; u++) {
        ks.compute(acc, ring[u]);
        ks.load_b(ring[u], boff, soff, s0 + u + R);
        ks.load_a(ring[u], s0 + u + R);
      }
      ks.pad();
    }
#pragma unroll
    for (int u = 0; u < 2 * R; u++) {
      const int s = s0 + u;
      if (s < n) {
        ks.compute(acc, ring[u % R]);
        ks.pad();
        if (s + R < n) {
          ks.load_b(ring[u % R], boff, soff, s + R);
          ks.load_a(ring[u % R], s + R);
        }
      }
    }
  } else {
    // Fewer steps than ring slots: every step's loads up front.
#pragma unroll
    for (int u = 0; u < R; u++)
      if (u < n) ks.load_b(ring[u], boff, soff, u);
    wait();
#pragma unroll
    for (int u = 0; u < R; u++)
      if (u < n) ks.load_a(ring[u], u);
#pragma unroll
    for (int u = 0; u < R; u++) {
      if (u < n) {
        ks.compute(acc, ring[u]);
        ks.pad();
      }
    }
  }
}

// The K loops of nch chunks of a unit's weight rows as one stream of loads
// (n a multiple of R; chunk c's rows start bchunk code bytes and schunk scale
// bytes after chunk c-1's): acc[s] += rows (16, A) x weight rows of sub-tile
// s over K steps 0..n-1, then epi(c, acc), for each chunk in turn.  Step s
// computes from ring[s % R] and then loads the step R later into it; the
// last R steps of a chunk load the next chunk's first R steps, so one
// chunk's epilogue overlaps the loads of the next, and those of the last
// chunk load nothing.
template <int S, bool PK, int R, int SRC, class Wait, class Epi>
__device__ inline void k_loop_chunks(const KStep<S, PK, SRC>& ks, const uint32_t (&boff)[2],
                                     const uint32_t (&soff)[2], uint32_t bchunk,
                                     uint32_t schunk, int n, int nch, Wait wait, Epi epi) {
  using Acc = typename Tr<S>::Acc;
  Slot<S> ring[R];
#pragma unroll
  for (int u = 0; u < R; u++) ks.load_b(ring[u], boff, soff, u);
  wait();
#pragma unroll
  for (int u = 0; u < R; u++) ks.load_a(ring[u], u);
  for (int c = 0; c < nch; c++) {
    Acc acc[2] = {Acc{0, 0, 0, 0}, Acc{0, 0, 0, 0}};
    const uint32_t bo[2] = {boff[0] + c * bchunk, boff[1] + c * bchunk};
    const uint32_t so[2] = {soff[0] + c * schunk, soff[1] + c * schunk};
    int s0 = 0;
    for (; s0 + R < n; s0 += R) {
#pragma unroll
      for (int u = 0; u < R; u++) {
        ks.compute(acc, ring[u]);
        ks.load_b(ring[u], bo, so, s0 + u + R);
        ks.load_a(ring[u], s0 + u + R);
      }
      ks.pad();
    }
    if (c + 1 < nch) {
      const uint32_t bn[2] = {bo[0] + bchunk, bo[1] + bchunk};
      const uint32_t sn[2] = {so[0] + schunk, so[1] + schunk};
#pragma unroll
      for (int u = 0; u < R; u++) {
        ks.compute(acc, ring[u]);
        ks.load_b(ring[u], bn, sn, u);
        ks.load_a(ring[u], u);
      }
    } else {
#pragma unroll
      for (int u = 0; u < R; u++) ks.compute(acc, ring[u]);
    }
    ks.pad();
    epi(c, acc);
  }
}

// Weight offsets of sub-tiles s = 0, 1 (weight rows nrow[s]; K elements per
// row K) in the streaming or canonical layout.
template <int S, bool PK>
__device__ inline void weight_offsets(const int (&nrow)[2], int K, uint32_t (&boff)[2],
                                      uint32_t (&soff)[2]) {
  using T_ = Tr<S>;
  constexpr int SB = (S == kW4A16 || S == kW4A8) ? 2 : 1;
  const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
  const uint32_t kbytes = (uint32_t)K * T_::KB_NUM / T_::KB_DEN;
#pragma unroll
  for (int s = 0; s < 2; s++) {
    if constexpr (PK) {
      const uint32_t g16 = (uint32_t)(nrow[s] - lr);
      boff[s] = g16 * kbytes + lane * 16;
      soff[s] = g16 * (uint32_t)(K / 32) * SB + (S == kW4A8 ? lr * 8 : lane * 2);
    } else {
      boff[s] = (uint32_t)nrow[s] * kbytes + lq * (S == kW4A8 ? 4 : T_::B_FRAG);
      soff[s] = (uint32_t)nrow[s] * (uint32_t)(K / 32) * SB + (S == kW4A8 ? 0 : lq * 2);
    }
  }
}

// Slot j's expert, row count and this lane's row (lane & 15): its pair, or
// the slot's last pair again for lanes past the rows (valid = false).
struct SlotRows {
  int e, nrows, pair;
  bool valid;
};

// Waits for slot j's record (wave 0 of the workgroup polls its copy and
// passes the record on through LDS; every wave of the workgroup belongs to
// slot j), reads it and counts the workgroup's pass; false if the slot
// holds no expert.  (The clamps only matter after a timed-out wait, when
// the record may be stale: every index then still stays inside its buffer.)
__device__ inline bool enter_slot(const DecodeArgs& g, int j, SlotRows& r, uint32_t* s_rec) {
  const int lane = threadIdx.x & 63;
  if (!g.local_route && (threadIdx.x >> 6) == 0) {
    int32_t* flag = &g.slot_flag[(blockIdx.x % kCopies) * g.smax + j];
    wait_set(flag, g);
    if (lane < 5) s_rec[lane] = (uint32_t)cload(&g.slot_rec[j * 8 + lane]);
    if (lane == 0) atomic_add(flag, -1);
  }
  __syncthreads();
  const uint32_t w1 = s_rec[0];
  const int n = (int)(w1 >> 16);
  if (n == 0) return false;
  const int lr = lane & 15;
  r.e = min((int)(w1 & 0xffffu), g.E - 1);
  r.nrows = min(n, kMaxTokens);
  r.valid = lr < r.nrows;
  const int row = r.valid ? lr : r.nrows - 1;  // lanes past the rows take the last row
  r.pair = min((int)((s_rec[1 + (row >> 2)] >> (8 * (row & 3))) & 0xffu), g.P - 1);
  return true;
}

template <int S, bool PK, int R>
__device__ void stage1_unit(const DecodeArgs& g, int j, int c, uint32_t* s_rec) {
  using T_ = Tr<S>;
  using Acc = typename T_::Acc;
  SlotRows sr;
  if (!enter_slot(g, j, sr, s_rec)) return;
  const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
  const int I = g.I, H = g.H, N = 2 * I;
  constexpr int SB = (S == kW4A16 || S == kW4A8) ? 2 : 1;
  const int nrow[2] = {c * 16 + lr, I + c * 16 + lr};
  uint32_t boff[2], soff[2];
  weight_offsets<S, PK>(nrow, H, boff, soff);
  const size_t kbytes = (size_t)H * T_::KB_NUM / T_::KB_DEN;
  const uint8_t* B = reinterpret_cast<const uint8_t*>(g.w13) + (size_t)sr.e * N * kbytes;
  const uint8_t* Sc =
      reinterpret_cast<const uint8_t*>(g.w13_scale) + (size_t)sr.e * N * (H / 32) * SB;
  const int tok = sr.pair / g.k;
  const uint8_t* arow = reinterpret_cast<const uint8_t*>(g.x) + (size_t)tok * H * T_::A_ELEM;
  Acc acc[2] = {Acc{0, 0, 0, 0}, Acc{0, 0, 0, 0}};
  k_loop<S, PK, R, kFromGlobal>(KStep<S, PK, kFromGlobal>(B, Sc, arow), boff, soff, H / T_::BK,
                                acc, [] {});

  // Epilogue: lane (lq, lr) holds rows 4lq + r of h column c*16 + lr.
  float ws[2] = {1.f, 1.f};
  if constexpr (S == kW8A8) {
#pragma unroll
    for (int s = 0; s < 2; s++)
      ws[s] = reinterpret_cast<const float*>(g.w13_scale)[(size_t)sr.e * N + nrow[s]];
  }
  const int col = c * 16 + lr;
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const int row = 4 * lq + r;
    const bool ok = row < sr.nrows;
    const int p = __shfl(sr.pair, row, 64);
    float gf, uf;
    if constexpr (S == kW8A8) {
      const float xs = g.x_scale[p / g.k];
      gf = ((float)acc[0][r] * xs) * ws[0];
      uf = ((float)acc[1][r] * xs) * ws[1];
    } else if constexpr (S == kA8W4 || S == kW4A8) {
      const float xs = g.x_scale[p / g.k];
      gf = acc[0][r] * xs;
      uf = acc[1][r] * xs;
    } else {
      gf = acc[0][r];
      uf = acc[1][r];
    }
    const float h = ok ? silu_mul<S>(gf, uf) : 0.f;
    if constexpr (S == kW4A16) {
      if (ok)
        cstore(reinterpret_cast<uint16_t*>(g.hq) + (size_t)p * I + col,
               __builtin_bit_cast(uint16_t, (__bf16)h));
    } else {
      if (ok) cstore(&g.h32[(size_t)p * I + col], h);
      const float a = group_max<16>(fabsf(h));
      if (ok && lr == 15) cstore(&g.pmax[(size_t)p * g.c1 + c], a);
    }
  }
  release();
  if (wave_add(&g.s1cnt[j], 1) != g.c1 - 1) return;

  // The slot's last stage-1 unit lets its stage-2 units go (they quantize
  // the slot's rows themselves; W4A16 passes h on in bf16).
  if (lane == 0) atomic_set(&g.s1cnt[j], 0);
  release();
  if (lane < kCopies) {
    const int b2 = stage2_block(g, j);
    const int n = count_mod(b2, b2 + g.c2 / kWaves, lane);
    if (n > 0) atomic_set(&g.ready[lane * g.smax + j], n);
  }
}

// out[t, c*32 + lane] for lanes 0..31: the combine's recipe (fp32, slot
// order j = 0..k-1, acc = acc + w*y without a fused multiply-add).
template <bool F32>
__device__ inline void combine_cols(const DecodeArgs& g, int t, int c, const float* lds_w) {
  const int lane = threadIdx.x & 63;
  if (lane >= 32) return;
  const int col = c * 32 + lane;
  float acc = 0.f;
  for (int j = 0; j < g.k; j++) {
    const size_t idx = ((size_t)t * g.k + j) * g.H + col;
    float v;
    if constexpr (F32)
      v = cload(reinterpret_cast<const float*>(g.y) + idx);
    else
      v = __uint_as_float((uint32_t)cload(reinterpret_cast<const uint16_t*>(g.y) + idx) << 16);
    const float wj = g.local_route ? lds_w[t * g.k + j] : cload(&g.topk_w[(size_t)t * g.k + j]);
    acc = acc + wj * v;
  }
  const size_t o = (size_t)t * g.H + col;
  if (g.out_f32 != nullptr) g.out_f32[o] = acc;
  if (g.out_bf16 != nullptr) g.out_bf16[o] = __builtin_bit_cast(uint16_t, (__bf16)acc);
}

template <int S, bool PK, int R>
__device__ void stage2_unit(const DecodeArgs& g, int j, int cg, uint32_t* s_rec,
                            const float* lds_w, uint8_t* qrows) {
  using T_ = Tr<S>;
  using Acc = typename T_::Acc;
  SlotRows sr;
  if (!enter_slot(g, j, sr, s_rec)) return;
  const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
  const int I = g.I, H = g.H;
  constexpr int SB = (S == kW4A16 || S == kW4A8) ? 2 : 1;
  const size_t kbytes = (size_t)I * T_::KB_NUM / T_::KB_DEN;
  const uint8_t* B = reinterpret_cast<const uint8_t*>(g.w2) + (size_t)sr.e * H * kbytes;
  const uint8_t* Sc =
      reinterpret_cast<const uint8_t*>(g.w2_scale) + (size_t)sr.e * H * (I / 32) * SB;
  // The A rows: W4A16's bf16 h straight from global memory (device-coherent
  // loads); the quantized schemes' rows from LDS, where the workgroup
  // quantizes them (qrows: nrows rows of I codes, pitch I + 16 so that the
  // fragment reads of 16 rows hit 16 different bank groups; qscale: their
  // scales).
  constexpr int SRC = S == kW4A16 ? kFromCoherent : kFromLds;
  const int qpitch = I + 16;
  float* const qscale = reinterpret_cast<float*>(qrows + kMaxTokens * qpitch);
  const uint8_t* arow =
      S == kW4A16 ? reinterpret_cast<const uint8_t*>(g.hq) + (size_t)sr.pair * I * T_::A_ELEM
                  : qrows + (size_t)min(lr, sr.nrows - 1) * qpitch;
  // This lane's rows (4lq + r) of the epilogue: pair and h row scale.
  int prow[4];
  float rsc[4] = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
  for (int r = 0; r < 4; r++) prow[r] = __shfl(sr.pair, 4 * lq + r, 64);
  const KStep<S, PK, SRC> ks(B, Sc, arow);
  const int n = I / T_::BK;
  // Wave 0 polls the workgroup's copy of the flag; then (quantized schemes)
  // the four waves requantize the slot's rows into LDS, wave w taking rows
  // w, w + 4, ...: the row scale from the maxima of its 16-column groups,
  // each group of four values to four codes (the recipe of the grouped
  // path's requantization), and the row scales for the epilogue.
  auto wait_ready = [&] {
    if ((threadIdx.x >> 6) == 0) {
      int32_t* f = &g.ready[(blockIdx.x % kCopies) * g.smax + j];
      wait_set(f, g);
      if (lane == 0) atomic_add(f, -1);
    }
    __syncthreads();
    if constexpr (S != kW4A16) {
      constexpr bool FP8 = S == kA8W4;
      const int wave = threadIdx.x >> 6;
      for (int r = wave; r < sr.nrows; r += kWaves) {
        const int p = __shfl(sr.pair, r, 64);
        const float* src = g.h32 + (size_t)p * I;
        uint32_t* dst = reinterpret_cast<uint32_t*>(qrows + r * qpitch);
        // The row maxima and the first 1024 values are loaded together.
        float a = 0.f;
        for (int i = lane; i < g.c1; i += 64) a = fmaxf(a, cload(&g.pmax[(size_t)p * g.c1 + i]));
        float v[4][4];
#pragma unroll
        for (int b = 0; b < 4; b++) {
          const int i = lane + 64 * b;
          if (i < I / 4) {
#pragma unroll
            for (int e = 0; e < 4; e++) v[b][e] = cload(src + 4 * i + e);
          }
        }
        a = wave_max(a);
        const float sc = rq::row_scale<FP8>(a);
        const bool refine = sc >= 0x1p-60f;
        const float rc = 1.0f / sc;
#pragma unroll
        for (int b = 0; b < 4; b++) {
          const int i = lane + 64 * b;
          if (i < I / 4) dst[i] = rq::quant4<FP8>(v[b][0], v[b][1], v[b][2], v[b][3], sc, rc, refine);
        }
        for (int i = lane + 256; i < I / 4; i += 64) {
          const float v0 = cload(src + 4 * i), v1 = cload(src + 4 * i + 1);
          const float v2 = cload(src + 4 * i + 2), v3 = cload(src + 4 * i + 3);
          dst[i] = rq::quant4<FP8>(v0, v1, v2, v3, sc, rc, refine);
        }
        if (lane == 0) qscale[r] = sc;
      }
      __syncthreads();
    }
  };
  auto load_rsc = [&] {
    if constexpr (S != kW4A16) {
#pragma unroll
      for (int r = 0; r < 4; r++)
        if (4 * lq + r < sr.nrows) rsc[r] = qscale[4 * lq + r];
    }
  };
  // W8A8's per-column weight scales of 32-column chunk c.
  auto load_ws = [&](int c, float (&ws)[2]) __attribute__((always_inline)) {
    if constexpr (S == kW8A8) {
#pragma unroll
      for (int s = 0; s < 2; s++)
        ws[s] = reinterpret_cast<const float*>(g.w2_scale)[(size_t)sr.e * H + c * 32 + 16 * s + lr];
    }
  };
  // y of 32-column chunk c: lane (lq, lr) holds rows 4lq + r of columns
  // c*32 + 16s + lr.
  auto store = [&](int c, const Acc(&acc)[2], const float (&ws)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 4; r++) {
      if (4 * lq + r < sr.nrows) {
        const float rs = rsc[r];
#pragma unroll
        for (int s = 0; s < 2; s++) {
          const size_t o = (size_t)prow[r] * H + c * 32 + 16 * s + lr;
          if constexpr (S == kW8A8)
            cstore(reinterpret_cast<float*>(g.y) + o, ((float)acc[s][r] * rs) * ws[s]);
          else if constexpr (S == kA8W4 || S == kW4A8)
            cstore(reinterpret_cast<uint16_t*>(g.y) + o,
                   __builtin_bit_cast(uint16_t, (__bf16)(acc[s][r] * rs)));
          else
            cstore(reinterpret_cast<uint16_t*>(g.y) + o,
                   __builtin_bit_cast(uint16_t, (__bf16)acc[s][r]));
        }
      }
    }
  };
  if (g.G > 1 && n % R == 0) {
    // The unit's chunks as one stream of loads.  The row scales are loaded
    // right after the flag (before the activation loads, so no wait for them
    // holds up the K loop); each chunk's weight scales are loaded during the
    // previous chunk's epilogue, long before they are used.
    const int c0 = cg * g.G;
    const int nrow[2] = {c0 * 32 + lr, c0 * 32 + 16 + lr};
    uint32_t boff[2], soff[2];
    weight_offsets<S, PK>(nrow, I, boff, soff);
    float ws[2] = {1.f, 1.f};
    load_ws(c0, ws);
    k_loop_chunks<S, PK, R, SRC>(
        ks, boff, soff, 32u * (uint32_t)kbytes, (uint32_t)I * SB, n, g.G,
        [&] {
          wait_ready();
          load_rsc();
        },
        [&](int c, const Acc(&acc)[2]) __attribute__((always_inline)) {
          store(c0 + c, acc, ws);
          if (c + 1 < g.G) load_ws(c0 + c + 1, ws);
        });
  } else {
    auto chunk = [&](int c, bool first) __attribute__((always_inline)) {
      const int nrow[2] = {c * 32 + lr, c * 32 + 16 + lr};
      uint32_t boff[2], soff[2];
      weight_offsets<S, PK>(nrow, I, boff, soff);
      Acc acc[2] = {Acc{0, 0, 0, 0}, Acc{0, 0, 0, 0}};
      if (first) {
        k_loop<S, PK, R, SRC>(ks, boff, soff, n, acc, wait_ready);
        load_rsc();
      } else {
        k_loop<S, PK, R, SRC>(ks, boff, soff, n, acc, [] {});
      }
      float ws[2] = {1.f, 1.f};
      load_ws(c, ws);
      store(c, acc, ws);
    };
    chunk(cg * g.G, true);
    for (int gi = 1; gi < g.G; gi++) chunk(cg * g.G + gi, false);
  }
  release();
  // One arrival per row (lanes 0..15 hold rows 0..15); the last of a token's
  // k rows to arrive for this unit's columns combines them.
  bool last = false;
  if (lane < 16 && sr.valid) {
    int32_t* cp = &g.ccnt[(sr.pair / g.k) * g.c2 + cg];
    last = atomic_add(cp, 1) == g.k - 1;
    if (last) atomic_set(cp, 0);
  }
  uint64_t mask = __ballot(last);
  if (mask == 0) return;
  acquire();
  while (mask != 0) {
    const int r = __builtin_ctzll(mask);
    mask &= mask - 1;
    const int t = __shfl(sr.pair, r, 64) / g.k;
    for (int gi = 0; gi < g.G; gi++) combine_cols<S == kW8A8>(g, t, cg * g.G + gi, lds_w);
  }
}

template <int S, bool PK, int R>
__global__ __launch_bounds__(kWaves * 64) void decode_kernel(DecodeArgs g) {
  __shared__ AlignLds lds;
  __shared__ uint32_t s_rec[8];
  // Quantized schemes: a stage-2 workgroup's requantized slot rows and
  // their scales (decode_lds_bytes).
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];
  // The workgroup's four units: all routing units, or four column chunks of
  // one slot in one stage (u0, c1 and c2 are multiples of four).
  const int u = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (u < g.u0) {
    if (u < g.T) route_unit(g, u, lds);
    return;
  }
  int v = u - g.u0;
  const int n1 = g.smax * g.c1;
  if (g.local_route) {
    // The workgroup's slot (the same for its four units).
    const int vb = blockIdx.x * kWaves - g.u0;
    route_local(g, lds, vb < n1 ? vb / g.c1 : (vb - n1) / g.c2, s_rec);
  }
  if (v < n1) {
    stage1_unit<S, PK, R>(g, v / g.c1, v % g.c1, s_rec);
    return;
  }
  v -= n1;
  if (v < g.smax * g.c2) stage2_unit<S, PK, R>(g, v / g.c2, v % g.c2, s_rec, lds.wts, dyn_lds);
}

}  // namespace

int decode_max_tokens() { return kMaxTokens; }

// Workspace layout (byte offsets), sized for kMaxTokens tokens so that one
// zeroed workspace serves every batch size of the same layer shape.  The
// counters come first (decode_counter_bytes of them must be zero before the
// first call).
DecodeWs decode_ws_layout(int scheme, int H, int I, int E, int k) {
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  const size_t P = (size_t)kMaxTokens * k;
  const size_t smax = std::min<size_t>((size_t)E, P);
  const size_t c2 = (size_t)H / 32, c1 = (size_t)I / 16;
  DecodeWs w{};
  size_t off = 0;
  w.flags = off;
  off = up(off + 4);
  w.route_cnt = off;
  off = up(off + 4);
  w.slot_flag = off;
  off = up(off + kCopies * smax * 4);
  w.slot_rec = off;
  off = up(off + smax * 32);
  w.s1cnt = off;
  off = up(off + smax * 4);
  w.ready = off;
  off = up(off + kCopies * smax * 4);
  w.ccnt = off;
  off = up(off + (size_t)kMaxTokens * c2 * 4);
  w.counter_bytes = off;
  const bool w4a16 = scheme == kW4A16;
  if (!w4a16) {
    w.h32 = off;
    off = up(off + P * I * 4);
    w.pmax = off;
    off = up(off + P * c1 * 4);
  } else {
    w.hq = off;
    off = up(off + P * I * 2);
  }
  w.y = off;
  off = up(off + P * H * (scheme == kW8A8 ? 4 : 2));
  w.total = off;
  return w;
}

template <int S, bool PK, int R>
static hipError_t launch_t(const DecodeArgs& g, unsigned blocks, hipStream_t s) {
  const size_t dyn = S == kW4A16 ? 0 : (size_t)kMaxTokens * (g.I + 16 + 4);
  hipLaunchKernelGGL((decode_kernel<S, PK, R>), dim3(blocks), dim3(kWaves * 64), dyn, s, g);
  return hipGetLastError();
}

template <int S>
static hipError_t launch_s(const DecodeArgs& g, bool packed, int ring, unsigned blocks,
                           hipStream_t s) {
  if (packed)
    return ring == 6 ? launch_t<S, true, 6>(g, blocks, s) : launch_t<S, true, 4>(g, blocks, s);
  return ring == 6 ? launch_t<S, false, 6>(g, blocks, s) : launch_t<S, false, 4>(g, blocks, s);
}

// 32-column chunks per stage-2 unit.  More chunks per unit amortize its
// fixed costs (the flag, the activation reads, the arrival counts) over more
// weight bytes; fewer leave more units to fill the chip.  Measured on the
// 512-expert top-10 block (hidden 4096, 128 columns of 32): 1 chunk best at
// 1 token (1280 one-chunk units), 2 at 2-8 tokens, 4 at 16 tokens (4800
// four-chunk units); 8 never.  So: 4 chunks when that still leaves 4096
// units, else 2 when one-chunk units would number 2048 or more, else 1 (and
// always a multiple of four units per slot).
int decode_stage2_chunks(int T, int H, int E, int k) {
  const long units1 = (long)std::min(E, T * k) * (H / 32);
  if ((H / 32) % 16 == 0 && units1 / 4 >= 4096) return 4;
  if ((H / 32) % 8 == 0 && units1 >= 2048) return 2;
  return 1;
}

hipError_t launch_decode(int scheme, bool packed, int ring, int chunks, int T, int H, int I,
                         int E, int k,
                         const float* logits, const void* x, const float* x_scale,
                         const void* w13, const void* w13_scale, const void* w2,
                         const void* w2_scale, int32_t* topk_ids, float* topk_w, void* y,
                         uint16_t* out_bf16, float* out_f32, void* ws, uint64_t spin_ticks,
                         hipStream_t s) {
  const DecodeWs L = decode_ws_layout(scheme, H, I, E, k);
  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  DecodeArgs g{};
  g.T = T, g.H = H, g.I = I, g.E = E, g.k = k, g.P = T * k;
  g.smax = std::min(E, T * k);
  g.c1 = I / 16;
  g.G = chunks;
  g.c2 = H / 32 / g.G;
  // Local routing up to 2 tokens: 1 token 45.8 -> 44.3 us, 2 tokens 61.4 ->
  // 60.5 us; at 4 tokens every workgroup routing four tokens before it starts
  // costs more than the hand-off (87.7 -> 94.4 us).
  g.local_route = T <= 2 ? 1 : 0;
  g.u0 = g.local_route ? 0 : (T + kWaves - 1) / kWaves * kWaves;
  g.logits = logits, g.x = x, g.x_scale = x_scale;
  g.w13 = w13, g.w13_scale = w13_scale, g.w2 = w2, g.w2_scale = w2_scale;
  g.topk_ids = topk_ids, g.topk_w = topk_w;
  g.y = y != nullptr ? y : base + L.y;
  g.out_bf16 = out_bf16, g.out_f32 = out_f32;
  g.flags = reinterpret_cast<int32_t*>(base + L.flags);
  g.route_cnt = reinterpret_cast<int32_t*>(base + L.route_cnt);
  g.slot_rec = reinterpret_cast<int32_t*>(base + L.slot_rec);
  g.slot_flag = reinterpret_cast<int32_t*>(base + L.slot_flag);
  g.s1cnt = reinterpret_cast<int32_t*>(base + L.s1cnt);
  g.ready = reinterpret_cast<int32_t*>(base + L.ready);
  g.ccnt = reinterpret_cast<int32_t*>(base + L.ccnt);
  g.h32 = scheme == kW4A16 ? nullptr : reinterpret_cast<float*>(base + L.h32);
  g.pmax = scheme == kW4A16 ? nullptr : reinterpret_cast<float*>(base + L.pmax);
  g.hq = scheme == kW4A16 ? base + L.hq : nullptr;
  g.spin_ticks = spin_ticks;
  const long units = (long)g.u0 + (long)g.smax * (g.c1 + g.c2);
  const unsigned blocks = (unsigned)((units + kWaves - 1) / kWaves);
  switch (scheme) {
    case kW4A16: return launch_s<kW4A16>(g, packed, ring, blocks, s);
    case kW8A8: return launch_s<kW8A8>(g, packed, ring, blocks, s);
    case kA8W4: return launch_s<kA8W4>(g, packed, ring, blocks, s);
    case kW4A8: return launch_s<kW4A8>(g, packed, ring, blocks, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qmoe
