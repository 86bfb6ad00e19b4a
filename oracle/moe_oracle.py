"""Plain, slow, fp64 CPU oracle of the grouped, weight-quantized MoE FFN.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module.  It shares
no code with the HIP library: it reads the canonical input bytes and decodes
them itself.  NumPy only (matrix products are the one library primitive used).

What is computed, step by step:

1. Routing.  Softmax over fp32 router logits, the k largest (ties go to the
   lower expert index), weights renormalised over the k picked.  The pages
   name top-k routing (vLLM issue "Evaluate native IU4/IU8 WMMA for
   grouped-INT MoE prefill on gfx1151", section Problem; aiter PR 6090,
   section Changes: topk 10); the tie rule and the renormalisation are the
   problem statement's.  Renormalised softmax over the picked k equals the
   softmax of the picked logits, because the full denominator cancels.
2. Grouping.  (token, slot) pairs ``p = t*k + j`` sorted by expert, ascending
   pair id inside an expert, each non-empty expert padded with the sentinel
   ``P`` to a multiple of the tile height ``block_m``; one tile-to-expert
   entry per tile.  This is the batching of all experts' rows into one launch
   per projection of hip-ep PR "perf(qmoe): group prefill expert matmuls"
   (description), with the order fixed so results compare bit for bit.
3. Stage 1 per pair: ``gu = x[t] . W13[e]^T`` (rows 0..I-1 gate, I..2I-1 up).
4. ``h = silu(gate) * up`` with ``silu(g) = g / (1 + exp(-g))``, then h is
   stored in the scheme's activation format (bf16; int8 or fp8 e4m3 with a
   per-row absmax scale).
5. Stage 2 per pair: ``y = h . W2[e]^T`` (aiter PR 6090, Test Plan: stage1
   tiles, then stage2 tiles).
6. Combine: ``out[t] = sum_j w[t, j] * y[t*k + j]`` in slot order, a fixed
   order with no atomics (hip-ep PR, description: deterministic scatter order).

Schemes: ``w4a16`` (the int4 weights dequantised to bf16, q * s rounded to
nearest even, as the vLLM issue lowers W4A16, sections Problem and
Constraint; then exact fp64 arithmetic),
``w4a8`` (int4 weights upconverted for an integer product with int8
activations: exact integer sums per 32-wide group, the group scales applied
after them, exact in fp64; the int8 requantization of h decided in fp32 as
for w8a8; vLLM issue, section Constraint: W4A8 with the weights upconverted
to 8 bits before the integer MMA),
``w8a8`` (exact integer accumulators; a fixed fp32 recipe for the rescales,
the SiLU and the requantization so the integer results can be compared bit
for bit), ``a8w4`` (the fp8 x e2m1 x 2^s products are exact in fp64 at these
sizes; the fp8 requantization of h is decided in fp32 like the kernels).

Pins (``tests/test_oracle.py``; every function below has at least one):
format decoders and encoders against torch's float8/e8m0/bf16 casts and the
OCP tables in ``tests/golden``; routing against a brute-force sort; grouping
against a brute-force stable sort and its invariants; one expert with top-1
against a textbook dense FFN; every expert on every token then select, against
the grouped layer; W8A8 accumulators against Python integers and the W8A8
rescale (``rescale_w8a8``) and the layer's gu and y against exact rationals
rounded to fp32 after each product; a8w4 accumulators against exact
rationals; the int8 and e4m3 requantization at exact ties where only the
correctly rounded quotient h / s gives the right code; SiLU closed forms;
``rel_l2`` closed forms.
"""
from __future__ import annotations

import numpy as np

f32 = np.float32
f64 = np.float64

# ----------------------------------------------------------------------------
# Number formats (decoders and encoders written from the format definitions)
# ----------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 is the upper half of an IEEE binary32 pattern."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(f64)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round finite values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits; with ``x = m * 2^e`` and
    ``0.5 <= |m| < 1`` the result is ``rint(m * 2^8) * 2^(e - 8)``.  Values
    below the normal range keep the fixed subnormal step 2^-133.
    """
    x = np.asarray(x, f64)
    m, e = np.frexp(x)
    e = np.maximum(e, -125)  # subnormal bf16 values share the 2^-133 step
    step = np.ldexp(1.0, e - 8)
    return np.rint(x / step) * step


def bf16_bits_from_value(v: np.ndarray) -> np.ndarray:
    """Bit pattern of values that are already exact bfloat16 values."""
    return (np.asarray(v, f64).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def int4_values(packed: np.ndarray) -> np.ndarray:
    """Two's-complement nibbles, two per byte, low nibble = even index."""
    p = np.asarray(packed, np.uint8)
    lo = (p & 0x0F).astype(np.int64)
    hi = (p >> 4).astype(np.int64)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    return np.stack([lo, hi], axis=-1).reshape(p.shape[:-1] + (2 * p.shape[-1],))


def _e2m1_value(code: int) -> float:
    """OCP MX FP4 (E2M1): 1 sign, 2 exponent (bias 1), 1 mantissa bit."""
    s = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        return s * (m * 0.5)  # subnormal: m/2 * 2^(1-1)
    return s * (1.0 + m * 0.5) * 2.0 ** (e - 1)


E2M1_TABLE = np.array([_e2m1_value(c) for c in range(16)], f64)


def e2m1_values(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, np.uint8)
    codes = np.stack([p & 0x0F, p >> 4], axis=-1).reshape(p.shape[:-1] + (2 * p.shape[-1],))
    return E2M1_TABLE[codes]


def e8m0_values(b: np.ndarray) -> np.ndarray:
    """OCP MX shared scale: 2^(b - 127); 0xFF is NaN."""
    b = np.asarray(b, np.uint8).astype(np.int64)
    v = np.ldexp(1.0, b - 127)
    return np.where(b == 255, np.nan, v)


def _e4m3_value(code: int) -> float:
    """OCP FP8 E4M3: 1 sign, 4 exponent (bias 7), 3 mantissa; S.1111.111 is NaN."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], f64)
E4M3_MAX = 448.0


def e4m3_values(codes: np.ndarray) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, np.uint8)]


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code, ties to even, magnitudes above 448 saturate to 448."""
    v = np.asarray(v, f64)
    sign = np.where(np.signbit(v), 0x80, 0x00).astype(np.int64)
    a = np.minimum(np.abs(v), E4M3_MAX)
    # Subnormal range (|v| < 2^-6): fixed step 2^-9, code = multiple of the step.
    sub_q = np.rint(a / 2.0 ** -9).astype(np.int64)  # may reach 8 == 2^-6 (code 8)
    # Normal range: |v| = (1 + q/8) * 2^E with E = floor(log2 |v|).
    m, e = np.frexp(np.where(a > 0, a, 1.0))  # a = m * 2^e, m in [0.5, 1)
    E = e - 1
    q = np.rint((a / np.ldexp(1.0, E) - 1.0) * 8.0).astype(np.int64)
    carry = q == 8
    E = np.where(carry, E + 1, E)
    q = np.where(carry, 0, q)
    normal_code = ((E + 7) << 3) | q
    code = np.where(a < 2.0 ** -6, sub_q, normal_code)
    return (code | sign).astype(np.uint8)


# ----------------------------------------------------------------------------
# Step 1: routing
# ----------------------------------------------------------------------------


def route(logits: np.ndarray, k: int):
    """Top-k experts per token and renormalised softmax weights.

    Slots are in descending logit order, ties to the lower expert index.
    ``w[t, j] = exp(L[e_j] - L[e_0]) / sum_i exp(L[e_i] - L[e_0])`` in fp64,
    stored as fp32.
    """
    L = np.asarray(logits, np.float32)
    T, E = L.shape
    assert 1 <= k <= E
    order = np.argsort(-L, axis=1, kind="stable")  # stable: equal logits keep index order
    ids = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(L, ids.astype(np.int64), axis=1).astype(f64)
    ex = np.exp(sel - sel[:, :1])
    den = np.zeros(T, f64)
    for j in range(k):  # denominator summed in slot order
        den = den + ex[:, j]
    w = (ex / den[:, None]).astype(np.float32)
    return ids, w


# ----------------------------------------------------------------------------
# Step 2: grouping by expert, padded to the tile height
# ----------------------------------------------------------------------------


def align(topk_ids: np.ndarray, E: int, block_m: int) -> dict:
    """Expert-major order of the pair ids, each expert padded to ``block_m``.

    Returns ``sorted_pair_ids`` (length ``num_padded``, sentinel = P),
    ``tile_expert`` (length ``num_padded / block_m``), ``expert_offsets``
    (E + 1 entries) and ``num_padded``.  Ids outside [0, E) are dropped.
    """
    ids = np.asarray(topk_ids, np.int64).reshape(-1)
    P = ids.size
    offsets = [0]
    order = []
    tiles = []
    for e in range(E):
        pairs = [p for p in range(P) if ids[p] == e]  # ascending pair id
        c = len(pairs)
        padded = -(-c // block_m) * block_m
        order.extend(pairs + [P] * (padded - c))
        tiles.extend([e] * (padded // block_m))
        offsets.append(offsets[-1] + padded)
    return {
        "sorted_pair_ids": np.array(order, np.int32),
        "tile_expert": np.array(tiles, np.int32),
        "expert_offsets": np.array(offsets, np.int32),
        "num_padded": int(offsets[-1]),
    }


# ----------------------------------------------------------------------------
# Weight decoding
# ----------------------------------------------------------------------------


def dequant_int4_g32(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """W[n, c] = q[n, c] * s[n, c // 32] (exact in fp64)."""
    q = int4_values(codes).astype(f64)
    s = np.repeat(np.asarray(scales).astype(f64), 32, axis=-1)
    return q * s


def dequant_mxfp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """W[n, c] = e2m1(q[n, c]) * 2^(S[n, c // 32] - 127) (exact in fp64)."""
    return e2m1_values(codes) * np.repeat(e8m0_values(scales), 32, axis=-1)


# ----------------------------------------------------------------------------
# Steps 3-5: one expert on a set of rows
# ----------------------------------------------------------------------------


def silu_mul_f32(gu: np.ndarray, inter: int) -> np.ndarray:
    """fp32 recipe: ex = f32(exp_f64(-g)); sg = g / (1 + ex); h = sg * u."""
    g = gu[:, :inter].astype(f32)
    u = gu[:, inter:].astype(f32)
    with np.errstate(over="ignore"):
        ex = np.exp(-g.astype(f64)).astype(f32)
    den = (f32(1.0) + ex).astype(f32)
    sg = (g / den).astype(f32)
    return (sg * u).astype(f32)


def quant_rows_int8(h: np.ndarray):
    """Per-row symmetric int8: s = f32(absmax / 127) (1 for an all-zero row),
    code = round-half-even(f32(h / s)) clamped to [-127, 127]."""
    h = np.asarray(h, f32)
    a = np.abs(h).max(axis=1)
    sh = np.where(a > 0, (a / f32(127.0)).astype(f32), f32(1.0)).astype(f32)
    hq = np.clip(np.rint((h / sh[:, None]).astype(f32)), -127, 127).astype(np.int64)
    return hq, sh


def quant_rows_e4m3(h: np.ndarray):
    """Per-row fp8: s = f32(absmax / 448) (1 for an all-zero row),
    code = e4m3_encode(f32(h / s))."""
    h = np.asarray(h, f32)
    a = np.abs(h).max(axis=1)
    sh = np.where(a > 0, (a / f32(448.0)).astype(f32), f32(1.0)).astype(f32)
    return e4m3_encode((h / sh[:, None]).astype(f32)), sh


def expert_w4a16(x_bits, w13, s13, w2, s2) -> dict:
    """The W4A16 lowering the vLLM issue describes (section Problem and
    Constraint): the packed int4 weights are dequantised to bf16 (q * s
    rounded to nearest even), then a bf16 dot, here with exact fp64 sums."""
    inter = w13.shape[0] // 2
    x = bf16_bits_to_f64(x_bits)
    gu = x @ round_to_bf16(dequant_int4_g32(w13, s13)).T
    g, u = gu[:, :inter], gu[:, inter:]
    with np.errstate(over="ignore"):
        h = g / (1.0 + np.exp(-g)) * u
    hin = round_to_bf16(h)
    y = hin @ round_to_bf16(dequant_int4_g32(w2, s2)).T
    return {"gu": gu, "h": hin, "y": y}


def rescale_w8a8(acc: np.ndarray, s_row: np.ndarray, s_col: np.ndarray) -> np.ndarray:
    """fp32 rescale of exact int32 sums: ``f32(f32(f32(acc) * s_row) * s_col)``,
    three roundings in this order (row = token or h row, col = output
    channel).  ``acc`` stays below 2^24 in magnitude here, so ``f32(acc)`` is
    exact; the two products are each rounded to nearest even."""
    a = np.asarray(acc).astype(f32)
    t = (a * np.asarray(s_row, f32)[:, None]).astype(f32)
    return (t * np.asarray(s_col, f32)[None, :]).astype(f32)


def expert_w8a8(xq, sx, w13, s13, w2, s2) -> dict:
    inter = w13.shape[0] // 2
    # int8 x int8 products summed over K < 2^31: integer-valued fp64 partial
    # sums stay exact (< 2^53), so the fp64 product is the exact integer.
    acc1 = np.rint(np.asarray(xq, f64) @ np.asarray(w13, f64).T).astype(np.int64)
    gu = rescale_w8a8(acc1, sx, s13)
    h = silu_mul_f32(gu, inter)
    hq, sh = quant_rows_int8(h)
    acc2 = np.rint(hq.astype(f64) @ np.asarray(w2, f64).T).astype(np.int64)
    y = rescale_w8a8(acc2, sh, s2)
    return {"acc1": acc1, "gu": gu, "h": h, "hq": hq, "h_scale": sh, "acc2": acc2, "y": y}


def expert_a8w4(xq, sx, w13, s13, w2, s2) -> dict:
    inter = w13.shape[0] // 2
    xv = e4m3_values(xq)
    acc1 = xv @ dequant_mxfp4(w13, s13).T  # exact: every partial sum fits 53 bits
    gu = (acc1.astype(f32) * np.asarray(sx, f32)[:, None]).astype(f32)
    h = silu_mul_f32(gu, inter)
    hq, sh = quant_rows_e4m3(h)
    acc2 = e4m3_values(hq) @ dequant_mxfp4(w2, s2).T
    y = acc2 * sh.astype(f64)[:, None]
    return {"acc1": acc1, "gu": gu, "h": h, "hq": hq, "h_scale": sh, "acc2": acc2, "y": y}


def group_sums_int4(xq: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """Exact integer dot products of int8 rows with int4 weight rows, one per
    32-wide group along K: ``acc[p, n, g] = sum_{c in group g} xq[p, c] *
    q[n, c]`` (fp64 products of integers below 2^53 are exact)."""
    x = np.asarray(xq, f64)
    q = int4_values(codes).astype(f64)
    P, K = x.shape
    N = q.shape[0]
    G = K // 32
    acc = np.empty((P, N, G), np.int64)
    for g in range(G):
        acc[:, :, g] = np.rint(x[:, 32 * g:32 * g + 32] @ q[:, 32 * g:32 * g + 32].T)
    return acc


def apply_group_scales(acc: np.ndarray, scales: np.ndarray, s_row: np.ndarray) -> np.ndarray:
    """``s_row[p] * sum_g s[n, g] * acc[p, n, g]`` in fp64: the group scales
    multiply the exact integer group sums.  The sum over groups is exact
    here: with fp16 scales in [2^-8, 2^-5) and |acc| < 2^15 every product is
    a multiple of 2^-18 below 2^10, and a sum of up to 128 of them stays
    below 2^17 (35 bits); the product with the fp32 row scale is then the
    one rounding (to fp64)."""
    sc = np.asarray(scales).astype(f64)  # [N, G]
    dot = np.einsum("png,ng->pn", acc.astype(f64), sc)
    return dot * np.asarray(s_row, f64)[:, None]


def expert_w4a8(xq, sx, w13, s13, w2, s2) -> dict:
    """int4 weights (fp16 scale per 32 along K) x int8 per-token activations.

    Integer group sums, group scales applied after them, the per-token
    scale last; gu rounded to fp32, then the fp32 SiLU recipe and the
    per-row int8 requantization of W8A8 (the scheme's activation format);
    stage 2 the same way with the row scale of h."""
    inter = w13.shape[0] // 2
    acc1 = group_sums_int4(xq, w13)
    gu = apply_group_scales(acc1, s13, sx).astype(f32)
    h = silu_mul_f32(gu, inter)
    hq, sh = quant_rows_int8(h)
    acc2 = group_sums_int4(hq, w2)
    y = apply_group_scales(acc2, s2, sh)
    return {"acc1": acc1, "gu": gu, "h": h, "hq": hq, "h_scale": sh, "acc2": acc2, "y": y}


def expert_ffn(scheme: str, x_rows, xs_rows, wts: dict) -> dict:
    if scheme == "w4a16":
        return expert_w4a16(x_rows, wts["w13"], wts["w13_scale"], wts["w2"], wts["w2_scale"])
    if scheme == "w8a8":
        return expert_w8a8(x_rows, xs_rows, wts["w13"], wts["w13_scale"], wts["w2"],
                           wts["w2_scale"])
    if scheme == "a8w4":
        return expert_a8w4(x_rows, xs_rows, wts["w13"], wts["w13_scale"], wts["w2"],
                           wts["w2_scale"])
    if scheme == "w4a8":
        return expert_w4a8(x_rows, xs_rows, wts["w13"], wts["w13_scale"], wts["w2"],
                           wts["w2_scale"])
    raise ValueError(scheme)


# ----------------------------------------------------------------------------
# Step 6: combine
# ----------------------------------------------------------------------------


def combine(scheme: str, y_pairs: np.ndarray, topk_w: np.ndarray) -> dict:
    """Slot-order weighted sum per token.

    w8a8: ``acc = f32(acc + f32(w * y))`` from 0, then bf16.  Others: the fp64
    sum (the reference value the bf16 output is measured against).
    """
    T, k = topk_w.shape
    y = y_pairs.reshape(T, k, -1)
    if scheme == "w8a8":
        acc = np.zeros((T, y.shape[-1]), f32)
        for j in range(k):
            acc = (acc + (topk_w[:, j:j + 1].astype(f32) * y[:, j].astype(f32)).astype(f32)) \
                .astype(f32)
        return {"out32": acc, "out": round_to_bf16(acc)}
    acc = np.zeros((T, y.shape[-1]), f64)
    for j in range(k):
        acc = acc + topk_w[:, j:j + 1].astype(f64) * y[:, j].astype(f64)
    return {"out": acc}


# ----------------------------------------------------------------------------
# Whole layer
# ----------------------------------------------------------------------------


def moe_forward(scheme: str, x, x_scale, weights, topk_ids, topk_w, keep=(),
                map_fn=map) -> dict:
    """Run the experts over all (token, slot) pairs and combine.

    ``weights`` is a dict of stacked ``[E, ...]`` arrays or a callable
    ``e -> dict`` for one expert.  ``keep`` names per-pair intermediates to
    return (e.g. ``("acc1", "acc2")``), indexed by pair id.  The experts are
    independent of one another; ``map_fn`` (the builtin ``map`` by default,
    or a thread pool's ``map``) runs them, and the results are placed in
    ascending expert order either way.
    """
    ids = np.asarray(topk_ids, np.int64)
    T, k = ids.shape
    P = T * k
    flat = ids.reshape(-1)
    y_pairs = None
    kept = {}

    def run_expert(e):
        pairs = np.nonzero(flat == e)[0]
        tok = pairs // k
        wts = weights(int(e)) if callable(weights) else {n: v[e] for n, v in weights.items()}
        xs_rows = None if x_scale is None else np.asarray(x_scale)[tok]
        r = expert_ffn(scheme, np.asarray(x)[tok], xs_rows, wts)
        return pairs, {n: r[n] for n in ("y",) + tuple(keep)}

    for pairs, r in map_fn(run_expert, np.unique(flat)):
        if y_pairs is None:
            y_pairs = np.zeros((P, r["y"].shape[1]), r["y"].dtype)
        y_pairs[pairs] = r["y"]
        for name in keep:
            v = r[name]
            if name not in kept:
                kept[name] = np.zeros((P,) + v.shape[1:], v.dtype)
            kept[name][pairs] = v
    res = combine(scheme, y_pairs, np.asarray(topk_w))
    res["y_pairs"] = y_pairs
    res.update(kept)
    return res


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    """||a - b||_2 / ||b||_2 over all elements, in fp64."""
    a = np.asarray(a, f64)
    b = np.asarray(b, f64)
    nb = np.linalg.norm(b.ravel())
    return float(np.linalg.norm((a - b).ravel()) / (nb if nb > 0 else 1.0))


__all__ = [
    "bf16_bits_to_f64", "round_to_bf16", "bf16_bits_from_value", "int4_values",
    "E2M1_TABLE", "e2m1_values", "e8m0_values", "E4M3_TABLE", "e4m3_values", "e4m3_encode",
    "route", "align", "quant_rows_int8", "quant_rows_e4m3", "silu_mul_f32", "dequant_int4_g32",
    "dequant_mxfp4", "rescale_w8a8", "group_sums_int4", "apply_group_scales", "expert_w4a16",
    "expert_w8a8", "expert_w4a8",
    "expert_a8w4", "expert_ffn", "combine", "moe_forward", "rel_l2",
]
