/*
 * qmoe.h -- C ABI of the grouped, weight-quantized Mixture-of-Experts FFN
 * for MI355X (gfx950).
 *
 * The layer: every token t picks k experts from its router logits; for each
 * (token, slot) pair p = t*k + j routed to expert e
 *     gu = x[t] . W13[e]^T          (W13 rows 0..I-1 = gate, I..2I-1 = up)
 *     h  = silu(gate) * up,  silu(g) = g / (1 + exp(-g))
 *     y[p] = h . W2[e]^T
 * and out[t] = sum_j w[t, j] * y[t*k + j] in slot order.
 *
 * Sources: hip-ep PR "perf(qmoe): group prefill expert matmuls" (description:
 * symmetric int4 expert projections batched into one launch per projection,
 * deterministic scatter order); vLLM issue "Evaluate native IU4/IU8 WMMA for
 * grouped-INT MoE prefill on gfx1151" (Problem: top-k routing, dequantise
 * then bf16 dot; Constraint: integer matrix products need an activation-
 * quantised scheme such as W8A8-int8); aiter PR 6090 (Changes: fp8
 * activations x MXFP4 weights, model_dim 4096, 512 experts, topk 10; Test
 * Plan: stage1 then stage2 tiles, K tiles no larger than inter_dim).  The
 * activation function, the routing tie rule and the combine order are not
 * spelled out on those pages; this library fixes them as stated above.
 *
 * Conventions for every call:
 *  - Every pointer argument is device memory owned by the caller.  The
 *    library never allocates, frees or keeps a pointer after it returns.
 *  - Every call is enqueued on `stream` (a hipStream_t; NULL = the null
 *    stream) and returns without waiting for the GPU, except
 *    qmoe_check_flags, which synchronises the stream.
 *  - Arguments are validated on the host before anything is launched; on an
 *    error nothing is enqueued and the status says why.  No C++ exception
 *    crosses this interface.  T = 0 is valid: qmoe_align still writes its
 *    (empty) outputs, the other calls enqueue nothing.
 *  - Layouts are row-major with K contiguous.  int4 and e2m1 values are
 *    packed two per byte, the even K index in the low nibble.
 */
#ifndef QMOE_H_
#define QMOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QMOE_ABI_VERSION 4

typedef enum {
  QMOE_OK = 0,
  QMOE_ERR_INVALID_ARG = 1, /* null pointer, bad size, workspace too small */
  QMOE_ERR_UNSUPPORTED = 2, /* valid, but no kernel built for this shape   */
  QMOE_ERR_HIP = 3          /* the HIP runtime reported an error           */
} qmoe_status;

/* Weight / activation schemes.
 * W4A16_G32:  x bf16 [T,H]; W int4 two's complement, one fp16 scale per 32
 *             values along K: scale [E,N,K/32].  Intermediate h is bf16.
 * W8A8_PERCHAN: x int8 [T,H] + fp32 per-token scale [T]; W int8 with one
 *             fp32 scale per output channel [E,N]; int32 accumulation.  h is
 *             requantized per row to int8 with an fp32 scale.
 * A8W4_MXFP4: x OCP fp8 e4m3 [T,H] + fp32 per-token scale [T]; W e2m1 with
 *             one e8m0 scale byte per 32 along K [E,N,K/32].  h is
 *             requantized per row to e4m3 with an fp32 scale.
 * W4A8_G32:   x int8 [T,H] + fp32 per-token scale [T]; W int4 two's
 *             complement with one fp16 scale per 32 along K [E,N,K/32]
 *             (8-byte aligned).  Each 32-wide group's int8 x int4 sum is
 *             exact, the group scale multiplies it, the token scale the
 *             total (vLLM issue, section Constraint: W4A8 with the weights
 *             upconverted to 8 bits before the integer MMA).  h is
 *             requantized per row to int8 with an fp32 scale.           */
typedef enum {
  QMOE_W4A16_G32 = 0,
  QMOE_W8A8_PERCHAN = 1,
  QMOE_A8W4_MXFP4 = 2,
  QMOE_W4A8_G32 = 3
} qmoe_scheme;

typedef enum { QMOE_DT_BF16 = 0, QMOE_DT_F32 = 1 } qmoe_dtype;

/* Debug flag for qmoe_grouped_ffn (W8A8 and W4A8): also write the
 * accumulators of both projections into the workspace (see
 * qmoe_grouped_ffn_debug_offsets): W8A8 the int32 sums; W4A8 the fp32 sum
 * over groups of group scale x exact group sum, before the token (stage 1)
 * or row (stage 2) scale.                                                 */
#define QMOE_FLAG_DUMP_ACC 1u
/* Flag for qmoe_grouped_ffn: the codes and scales of w13 and w2 are in the
 * streaming layout written by qmoe_prepack instead of the canonical one.  */
#define QMOE_FLAG_PREPACKED 2u

typedef struct {
  int32_t scheme;   /* qmoe_scheme                                        */
  int32_t T;        /* tokens                                             */
  int32_t H;        /* hidden size (K of stage 1, N of stage 2)           */
  int32_t I;        /* expert intermediate size                           */
  int32_t E;        /* number of experts                                  */
  int32_t k;        /* experts per token                                  */
  int32_t block_m;  /* rows per tile; must equal the one given qmoe_align */
  uint32_t flags;   /* QMOE_FLAG_*                                        */
} qmoe_ffn_desc;

/* Per-expert weights, stacked over experts (device pointers).
 * w13 [E, 2I, H] codes, w13_scale as the scheme says; w2 [E, H, I] codes,
 * w2_scale likewise.                                                     */
typedef struct {
  const void* w13;
  const void* w13_scale;
  const void* w2;
  const void* w2_scale;
} qmoe_weights;

/* ---------------------------------------------------------------------
 * qmoe_prepack -- rewrite one stacked weight tensor (codes [E,N,K] and its
 * scales, canonical layout) into the library's streaming layout, once, at
 * set-up time; qmoe_grouped_ffn reads it when QMOE_FLAG_PREPACKED is set.
 * It moves bytes only (the values are unchanged) and is not part of a
 * forward pass.  The pages fix no weight layout beyond the formats; this one
 * makes every 16-byte load of a 64-lane wave part of one contiguous 1 KiB
 * run and every scale load part of one 128-byte run.
 * Let S = weight bytes per row per K step (A8W4: 256 K = 128 B; W8A8: 128 K
 * = 128 B; W4A16: 128 K = 64 B), KB = bytes per row, G = n/16*16.
 * Codes: byte b of row n of expert e, with ks = b/S, r = b%S, i = r/64,
 *   q = (r%64)/16, c = r%16, goes to
 *   (e*N + G)*KB + ks*16*S + i*1024 + (16*q + n%16)*16 + c.
 *   W4A8 (S = 64) moves nibbles instead: the byte at
 *   (e*N + G)*KB + ks*1024 + (16*q + n%16)*16 + 4*j + b, for q, j, b in
 *   0..3, holds the code of K = 128*ks + 32*j + 8*q + b of row n in its low
 *   nibble and that of K + 4 in its high nibble.
 * Scales (R = scale bytes per row; 8 bytes per row per step in every
 *   scheme): for q = 0..3, row n and step ks, the two bytes at
 *   (e*N + G)*R + ks*128 + (16*q + n%16)*2 hold, for A8W4, the e8m0 bytes
 *   of the 32-K blocks 8*ks + q and 8*ks + 4 + q of the row (in that
 *   order); for W4A16, the fp16 scale of group 4*ks + q.  W4A8: the eight
 *   bytes at (e*N + G)*R + ks*128 + (n%16)*8 are the fp16 scales of groups
 *   4*ks .. 4*ks + 3 of row n.
 * W8A8 per-channel fp32 scales are copied unchanged (scales_out may be
 * NULL for W8A8, then nothing is copied).
 * codes_out / scales_out have the byte sizes of codes / scales and must not
 * overlap them.  Requires N % 16 == 0 and K a multiple of 256 (A8W4) or
 * 128 (W4A16, W8A8, W4A8).  QMOE_ERR_INVALID_ARG otherwise.              */
qmoe_status qmoe_prepack(int32_t scheme, int32_t E, int32_t N, int32_t K, const void* codes,
                         const void* scales, void* codes_out, void* scales_out, void* stream);

int qmoe_abi_version(void);
const char* qmoe_status_str(qmoe_status s);
/* Raw hipError_t of the last QMOE_ERR_HIP on the calling thread.          */
int qmoe_last_hip_error(void);

/* ---------------------------------------------------------------------
 * qmoe_route -- top-k routing from router logits.
 * Softmax over fp32 logits [T,E], the k largest logits per token (ties go
 * to the lower expert index) in descending order, weights renormalised
 * over the k picked: w[t,j] = exp(L[e_j]-L[e_0]) / sum_i exp(L[e_i]-L[e_0]),
 * evaluated in fp64 and stored as fp32.  (vLLM issue, section Problem:
 * top-k routing; aiter PR 6090, section Changes: topk 10.)
 * Out: topk_ids int32 [T,k], topk_w fp32 [T,k].  Requires 1 <= k <= E,
 * k <= 16 and E <= 1024; logits must be finite.                          */
qmoe_status qmoe_route(const float* logits, int32_t T, int32_t E, int32_t k,
                       int32_t* topk_ids, float* topk_w, void* stream);

/* ---------------------------------------------------------------------
 * qmoe_default_block_m -- the tile height (block_m) to give qmoe_align and
 * qmoe_grouped_ffn for a shape and token count: the gfx950 tile table's
 * entry for the shape's token bucket (built by a tile sweep with a bit-exact
 * accuracy gate, aiter PR 6090, section Test Plan), else a rule on the mean
 * rows per expert.  qmoe_grouped_ffn takes the rest of that table entry
 * (blocks, prefetch depth, column passes) when it is called with this
 * block_m; any block_m gives the same results bit for bit.  Returns 0 for
 * invalid arguments.  The environment variable QMOE_TILE
 * ("s1w=8,s1r=4,s1runs=1,s1lb=1,s2w=4,s2p=8,s2h=0,s2q=1", any subset)
 * overrides those other choices in qmoe_grouped_ffn for sweeps (s1runs: 0
 * strided items, 1 runs of row tiles, 2 row tiles dealt to the XCDs; s2q:
 * the resident stage 2's work queue off or on); a malformed or inapplicable
 * value makes qmoe_grouped_ffn return QMOE_ERR_INVALID_ARG.               */
int32_t qmoe_default_block_m(int32_t scheme, int32_t T, int32_t H, int32_t I, int32_t E,
                             int32_t k);

/* ---------------------------------------------------------------------
 * qmoe_align -- group the P = T*k (token, slot) pairs by expert.
 * sorted_pair_ids[cap]: for experts e = 0..E-1 in order, the pair ids
 *   p = t*k+j with topk_ids[t,j] == e in ascending order, then the sentinel
 *   P until the expert's segment is a multiple of block_m; experts with no
 *   pair get no segment.  Entries from num_padded to cap also hold P.
 * tile_expert[cap/block_m]: expert of each block_m-row tile, -1 past
 *   num_padded.
 * expert_offsets[E+1]: start of each expert's segment; [E] = num_padded.
 * num_padded[1]: total padded rows.
 * cap = qmoe_align_capacity(T,k,E,block_m) entries must be allocated.
 * A token's k ids must be distinct.  Ids outside [0,E) are dropped and set
 * bit 0 of the flag word in `ws`; an id repeated within a token sets bit 1
 * (one of its pairs is then lost).  Read the word with qmoe_check_flags.
 * block_m is 16, 32, 64 or 128; E <= 1024.
 * This is the batching of every expert's rows into one launch per
 * projection (hip-ep PR, description) with a fixed, stable order.        */
size_t qmoe_align_capacity(int32_t T, int32_t k, int32_t E, int32_t block_m);
size_t qmoe_align_workspace(int32_t T, int32_t k, int32_t E);
qmoe_status qmoe_align(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E,
                       int32_t block_m, int32_t* sorted_pair_ids, int32_t* tile_expert,
                       int32_t* expert_offsets, int32_t* num_padded, void* ws,
                       size_t ws_bytes, void* stream);
/* ---------------------------------------------------------------------
 * qmoe_route_align -- qmoe_route followed by qmoe_align, with the same
 * outputs bit for bit (topk_ids, topk_w, and the grouping with its flag word
 * in `ws`, qmoe_align_workspace(T,k,E) bytes, 256-byte aligned).  Up to 16
 * tokens both steps run in one launch of one block, for the decode regime,
 * where the number of dependent launches bounds the step (vLLM issue,
 * section Problem: decode is bound by weight streaming and dispatch count;
 * aiter PR 6090, section Changes: token bucket 1-256).  Larger batches take
 * the two launches of the separate calls.  Requirements and errors are those
 * of qmoe_route and qmoe_align together.                                  */
qmoe_status qmoe_route_align(const float* logits, int32_t T, int32_t E, int32_t k,
                             int32_t block_m, int32_t* topk_ids, float* topk_w,
                             int32_t* sorted_pair_ids, int32_t* tile_expert,
                             int32_t* expert_offsets, int32_t* num_padded, void* ws,
                             size_t ws_bytes, void* stream);

/* Copies the align flag word to host memory *flags_out (synchronises).  */
qmoe_status qmoe_check_flags(const void* align_ws, int32_t* flags_out, void* stream);

/* ---------------------------------------------------------------------
 * qmoe_align_noalloc -- qmoe_align for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same outputs, bit for bit, with no workspace
 * argument.  The workspace lives in a device array inside the library, of
 * QMOE_ALIGN_NOALLOC_MAX_BYTES per GPU, held from the library's load until
 * the process ends; the call itself allocates nothing.
 * flags: optional device int32 that receives the flag word qmoe_align
 *   leaves in its workspace (bit 0: an id outside [0,E); bit 1: an id
 *   repeated within a token); NULL to discard it.
 * Limit: qmoe_align_workspace(T, k, E) <= QMOE_ALIGN_NOALLOC_MAX_BYTES
 *   (up to 65024 tokens with 1024 experts, 130304 with 512, 260608 with
 *   256); larger sizes return QMOE_ERR_UNSUPPORTED and launch nothing.
 * All calls on one GPU share its array: calls that overlap in time on one
 * GPU (two streams, or two host threads) race and give undefined outputs;
 * calls ordered on one stream are safe.                                   */
#define QMOE_ALIGN_NOALLOC_MAX_BYTES (1u << 20)
qmoe_status qmoe_align_noalloc(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E,
                               int32_t block_m, int32_t* sorted_pair_ids,
                               int32_t* tile_expert, int32_t* expert_offsets,
                               int32_t* num_padded, int32_t* flags, void* stream);

/* ---------------------------------------------------------------------
 * qmoe_grouped_ffn -- stage 1 (gate/up projection of every expert in one
 * launch, fused silu(gate)*up epilogue), the scheme's requantization of h,
 * stage 2 (down projection of every expert in one launch).  aiter PR 6090,
 * Test Plan: stage1 and stage2 tiles; vLLM issue, sections Problem and
 * Constraint: dequantise-then-bf16-dot for W4A16, integer products for
 * W8A8.
 * x: see qmoe_scheme; x_scale fp32 [T] (NULL for W4A16).
 * sorted_pair_ids / tile_expert / num_padded: qmoe_align's outputs for the
 *   same T, k, E and block_m.
 * y_pairs: [T*k, H], row p = pair p, unweighted expert output; bf16 for
 *   W4A16, A8W4 and W4A8, fp32 for W8A8.
 * ws: workspace of at least qmoe_grouped_ffn_workspace(d) bytes, 256-byte
 *   aligned; its contents need no initialisation (the call's first kernel
 *   clears the work-queue counters the last one uses).  Calls that share a
 *   workspace must be ordered on one stream.
 * Requirements: H % 256 == 0, I % 128 == 0 (I % 256 for A8W4), k <= E;
 *   W4A8 scales 8-byte aligned;
 *   below 4 GiB each: x (T*H elements), the stage-2 activations (cap*I
 *   elements, cap = qmoe_align_capacity) and one expert's W13 or W2 codes.
 * Errors: QMOE_ERR_INVALID_ARG for null pointers, bad sizes or a short
 * workspace; QMOE_ERR_UNSUPPORTED for sizes outside the requirements.    */
size_t qmoe_grouped_ffn_workspace(const qmoe_ffn_desc* d);
/* Byte offsets inside ws of the 4-byte debug dumps written with
 * QMOE_FLAG_DUMP_ACC: acc1 [cap, 2I] and acc2 [cap, H], row = sorted slot.
 * Returns QMOE_ERR_INVALID_ARG unless the scheme is W8A8 or W4A8.       */
qmoe_status qmoe_grouped_ffn_debug_offsets(const qmoe_ffn_desc* d, size_t* acc1_off,
                                           size_t* acc2_off);
qmoe_status qmoe_grouped_ffn(const qmoe_ffn_desc* d, const void* x, const float* x_scale,
                             const qmoe_weights* w, const int32_t* sorted_pair_ids,
                             const int32_t* tile_expert, const int32_t* num_padded,
                             void* y_pairs, void* ws, size_t ws_bytes, void* stream);

/* Same as qmoe_grouped_ffn, and also records stage_events[0..3] (each a
 * hipEvent_t created by the caller) on the stream: before stage 1, after
 * stage 1, after the separate requantization of h (the same point as after
 * stage 1 where stage 2 quantizes h itself: W4A16, and the one-byte schemes
 * with I <= 1024), after stage 2.  For measuring each kernel inside a
 * timed run.                                                             */
qmoe_status qmoe_grouped_ffn_profiled(const qmoe_ffn_desc* d, const void* x,
                                      const float* x_scale, const qmoe_weights* w,
                                      const int32_t* sorted_pair_ids,
                                      const int32_t* tile_expert, const int32_t* num_padded,
                                      void* y_pairs, void* ws, size_t ws_bytes,
                                      void* const stage_events[4], void* stream);

/* ---------------------------------------------------------------------
 * qmoe_combine -- out[t,:] = sum_{j=0}^{k-1} topk_w[t,j] * y_pairs[t*k+j,:]
 * accumulated in fp32 in slot order j = 0..k-1 (acc = acc + w*y, no fused
 * multiply-add), one thread per output element group, no atomics, so the
 * result is bitwise reproducible (hip-ep PR, description: deterministic
 * scatter order).  y_pairs dtype: QMOE_DT_BF16 or QMOE_DT_F32.
 * out_bf16 [T,H] (round to nearest even) and/or out_f32 [T,H]; at least
 * one must be non-NULL when T > 0.  Requires H % 8 == 0.                 */
qmoe_status qmoe_combine(const void* y_pairs, int32_t y_dtype, const float* topk_w,
                         int32_t T, int32_t k, int32_t H, uint16_t* out_bf16,
                         float* out_f32, void* stream);

/* ---------------------------------------------------------------------
 * qmoe_decode -- the whole layer for a small batch in ONE launch: routing
 * as qmoe_route, the grouping of the pairs by expert, stage 1 with the
 * fused silu(gate)*up epilogue, the scheme's requantization of h, stage 2
 * and the weighted combine as qmoe_combine.  In the decode regime every
 * expert GEMM has at most a few rows and the step is bound by weight
 * streaming and by the number of dependent launches (vLLM issue, section
 * Problem; aiter PR 6090, section Changes: token bucket 1-256); the
 * kernel resolves the dependencies between the steps inside the launch.
 * topk_ids, topk_w, y_pairs, out_bf16 and out_f32 equal those of
 * qmoe_route -> qmoe_align -> qmoe_grouped_ffn -> qmoe_combine bit for bit.
 * d: scheme, T (1..QMOE_DECODE_MAX_TOKENS; 0 launches nothing), H, I, E, k
 *   (k <= 16) and flags (QMOE_FLAG_PREPACKED only) as for
 *   qmoe_grouped_ffn; block_m is not used.
 * logits fp32 [T,E]; x, x_scale and w as for qmoe_grouped_ffn.
 * topk_ids int32 [T,k], topk_w fp32 [T,k]: written (as qmoe_route).
 * y_pairs: optional [T*k, H] (bf16; fp32 for W8A8), row = pair: written
 *   when non-NULL (the workspace holds them otherwise).
 * out_bf16 / out_f32 [T,H]: at least one non-NULL.
 * ws: qmoe_decode_workspace(d) bytes, 256-byte aligned, ZEROED ONCE before
 *   its first use (it holds arrival counters; every call that completes
 *   leaves them zero, so the same workspace serves any number of calls
 *   ordered on one stream, for every T of the same H, I, E, k, scheme).
 *   Calls that overlap in time must not share a workspace.  Its flag word
 *   (qmoe_check_flags(ws, ...)) gets bit 2 if a wait inside the kernel ran
 *   out of time (100 ms; it cannot happen while the kernel's units run in
 *   launch order, and means the outputs are wrong and the workspace must be
 *   zeroed again).
 * Requirements as for qmoe_grouped_ffn.  QMOE_ERR_UNSUPPORTED for T above
 * QMOE_DECODE_MAX_TOKENS, E above 1024, or I above QMOE_DECODE_MAX_INTER
 * in the schemes with quantized activations (each stage-2 workgroup holds
 * 16 requantized h rows in LDS); QMOE_ERR_INVALID_ARG for null
 * pointers, a short workspace, bad sizes, flags other than
 * QMOE_FLAG_PREPACKED, a QMOE_DECODE_RING environment value other than 4
 * or 6 (the K loops' prefetch depth) or a QMOE_DECODE_G value other than
 * 1, 2, 4 or 8 dividing H / 128 (32-column chunks per stage-2 work unit);
 * both only change how the work is split, for measurements.             */
#define QMOE_DECODE_MAX_TOKENS 16
#define QMOE_DECODE_MAX_INTER 4096
size_t qmoe_decode_workspace(const qmoe_ffn_desc* d);
qmoe_status qmoe_decode(const qmoe_ffn_desc* d, const float* logits, const void* x,
                        const float* x_scale, const qmoe_weights* w, int32_t* topk_ids,
                        float* topk_w, void* y_pairs, uint16_t* out_bf16, float* out_f32,
                        void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* QMOE_H_ */
