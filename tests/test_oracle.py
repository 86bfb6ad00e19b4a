"""Pins of the CPU oracle against things other than itself.

Library conversions (torch's float8/e8m0/bf16 casts), published format
tables (tests/golden), closed forms, invariants, brute force on tiny inputs
and exact integer / rational arithmetic on slices.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from quantized_mixture_experts_moe_amd import synth
from quantized_mixture_experts_moe_amd.shapes import MoEShape, W4A16_TINY

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        c, v = line.split()
        rows.append((int(c, 16), float(v)))
    return rows


# ---------------------------------------------------------------- formats

def test_e2m1_table_matches_ocp_spec():
    for code, v in _read_table("ocp_e2m1_values.txt"):
        got = O.E2M1_TABLE[code]
        assert got == v and math.copysign(1, got) == math.copysign(1, v), (code, got, v)


def test_e4m3_points_match_ofp8_spec():
    for code, v in _read_table("ocp_e4m3_points.txt"):
        got = O.E4M3_TABLE[code]
        if math.isnan(v):
            assert math.isnan(got)
        else:
            assert got == v, (hex(code), got, v)


def test_e4m3_decode_matches_torch_all_codes():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = O.e4m3_values(np.arange(256, dtype=np.uint8))
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    m = ~np.isnan(ref)
    np.testing.assert_array_equal(got[m], ref[m])


def test_e4m3_encode_matches_torch_rne():
    rng = np.random.default_rng(5)
    finite = O.E4M3_TABLE[~np.isnan(O.E4M3_TABLE)]
    mids = (np.sort(np.unique(finite))[1:] + np.sort(np.unique(finite))[:-1]) / 2
    vals = np.concatenate([
        rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 0.01,
        rng.standard_normal(20000) * 30, finite, mids, [0.0, -0.0, 2.0 ** -10, 3 * 2.0 ** -10],
    ]).astype(np.float32)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.e4m3_encode(vals)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(vals[i], got[i], ref[i]) for i in bad[:5]]


def test_e4m3_encode_saturates():
    got = O.e4m3_encode(np.array([448.0, 449.0, 470.0, 1e9, -500.0]))
    np.testing.assert_array_equal(got, [0x7E, 0x7E, 0x7E, 0x7E, 0xFE])


def test_e8m0_matches_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    got = O.e8m0_values(np.arange(256, dtype=np.uint8))
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    m = ~np.isnan(ref)
    np.testing.assert_array_equal(got[m], ref[m])


def test_bf16_decode_and_round_match_torch():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(50000) * 10.0 ** rng.integers(-30, 30, 50000),
                        [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 2.0 ** -130,
                         3 * 2.0 ** -134, 0.0]]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16)
    np.testing.assert_array_equal(O.round_to_bf16(v), ref.double().numpy())
    bits = ref.view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(O.bf16_bits_to_f64(bits), ref.double().numpy())
    np.testing.assert_array_equal(O.bf16_bits_from_value(ref.double().numpy()), bits)


def test_int4_nibbles():
    got = O.int4_values(np.array([[0x8F, 0x70, 0x12]], np.uint8))
    np.testing.assert_array_equal(got, [[-1, -8, 0, 7, 2, 1]])
    allb = np.arange(256, dtype=np.uint8)[None, :]
    v = O.int4_values(allb).reshape(256, 2)
    for b in range(256):
        lo, hi = b & 15, b >> 4
        assert v[b, 0] == (lo if lo < 8 else lo - 16)
        assert v[b, 1] == (hi if hi < 8 else hi - 16)


# ---------------------------------------------------------------- routing

def _route_brute(L, k):
    T, E = L.shape
    ids = np.zeros((T, k), np.int64)
    w = np.zeros((T, k))
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(L[t, e]), e))[:k]
        ids[t] = order
        ex = [math.exp(float(L[t, e]) - float(L[t, order[0]])) for e in order]
        w[t] = [v / sum(ex) for v in ex]
    return ids, w


@pytest.mark.parametrize("T,E,k", [(7, 8, 2), (5, 16, 5), (3, 6, 6), (9, 4, 1)])
def test_route_brute_force(T, E, k):
    rng = np.random.default_rng(T * 100 + E)
    L = rng.standard_normal((T, E)).astype(np.float32)
    L[0, 1] = L[0, 3]  # a tie
    ids, w = O.route(L, k)
    ids_b, w_b = _route_brute(L, k)
    np.testing.assert_array_equal(ids, ids_b)
    np.testing.assert_allclose(w, w_b, rtol=2 ** -22, atol=0)


def test_route_invariants():
    L = np.random.default_rng(3).standard_normal((500, 64)).astype(np.float32)
    for k in (1, 2, 8, 64):
        ids, w = O.route(L, k)
        assert np.all(np.abs(w.astype(np.float64).sum(1) - 1) <= k * 2.0 ** -23)
        assert all(len(set(r)) == k for r in ids)
        if k == 1:
            assert np.all(w == 1.0)
        if k == 64:
            assert np.all(np.sort(ids, 1) == np.arange(64))
        # descending logits in slot order
        sel = np.take_along_axis(L, ids.astype(np.int64), 1)
        assert np.all(np.diff(sel, axis=1) <= 0)


def test_route_ties_pick_lower_index():
    L = np.zeros((2, 6), np.float32)
    L[1] = [1, 2, 2, 2, 0, 2]
    ids, w = O.route(L, 3)
    np.testing.assert_array_equal(ids, [[0, 1, 2], [1, 2, 3]])
    np.testing.assert_array_equal(w, np.full((2, 3), np.float32(1 / 3)))


def test_route_signed_zeros_tie():
    """-0 and +0 are equal logits, so they tie and the lower index wins."""
    L = np.array([[-0.0, 0.0, -0.0, 0.0, -1.0]], np.float32)
    ids, w = O.route(L, 3)
    np.testing.assert_array_equal(ids, [[0, 1, 2]])
    np.testing.assert_array_equal(w, np.full((1, 3), np.float32(1 / 3)))


# ---------------------------------------------------------------- align

def _align_brute(ids, E, bm):
    flat = list(np.asarray(ids).reshape(-1))
    P = len(flat)
    keyed = sorted((int(e), p) for p, e in enumerate(flat) if 0 <= e < E)
    out, tiles, offs = [], [], [0]
    for e in range(E):
        ps = [p for (ee, p) in keyed if ee == e]
        pad = (len(ps) + bm - 1) // bm * bm
        out += ps + [P] * (pad - len(ps))
        tiles += [e] * (pad // bm)
        offs.append(offs[-1] + pad)
    return out, tiles, offs


@pytest.mark.parametrize("T,k,E,bm", [(16, 2, 8, 4), (33, 3, 7, 16), (1, 1, 1, 32), (20, 4, 64, 8)])
def test_align_brute_force_and_invariants(T, k, E, bm):
    rng = np.random.default_rng(T + k + E)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    a = O.align(ids, E, bm)
    out, tiles, offs = _align_brute(ids, E, bm)
    np.testing.assert_array_equal(a["sorted_pair_ids"], out)
    np.testing.assert_array_equal(a["tile_expert"], tiles)
    np.testing.assert_array_equal(a["expert_offsets"], offs)
    P = T * k
    s = a["sorted_pair_ids"]
    assert sorted(s[s < P].tolist()) == list(range(P))
    assert np.all(a["expert_offsets"] % bm == 0)
    counts = np.bincount(ids.reshape(-1), minlength=E)
    for e in range(E):
        seg = s[a["expert_offsets"][e]:a["expert_offsets"][e + 1]]
        assert np.sum(seg < P) == counts[e]
        assert np.all(np.diff(seg[seg < P]) > 0)
        assert np.all(seg[counts[e]:] == P)


def test_align_drops_out_of_range_ids():
    ids = np.array([[0, 5], [1, -1]], np.int32)
    a = O.align(ids, 2, 2)
    np.testing.assert_array_equal(a["sorted_pair_ids"], [0, 4, 2, 4])


# ---------------------------------------------------------------- small layers

def _tiny(scheme, T=24, H=64, I=32, E=4, k=2, seed=7):
    sh = MoEShape(f"t_{scheme}", scheme, tokens=T, hidden=H, inter=I, experts=E, topk=k,
                  seed=seed)
    return sh, synth.make_inputs(sh)


def _dense_reference(scheme, inp, e, rows):
    """Textbook dense FFN of one expert with torch ops, decoding the weights
    with torch's own format conversions where torch has them."""
    I = inp["w13"].shape[1] // 2
    H = inp["w2"].shape[1]
    if scheme == "w4a16":
        x = torch.from_numpy(inp["x"][rows].view(np.int16)).view(torch.bfloat16).double()

        def deq(codes, s):
            b = torch.from_numpy(codes.astype(np.int16))
            lo = (b & 15) - 16 * ((b & 15) >= 8).to(torch.int16)
            hi = (b >> 4) - 16 * ((b >> 4) >= 8).to(torch.int16)
            q = torch.stack([lo, hi], -1).reshape(codes.shape[0], -1).double()
            w = q * torch.from_numpy(s.astype(np.float64)).repeat_interleave(32, 1)
            # dequantised to bf16 (torch's round-to-nearest-even cast; q * s is
            # exact in fp32)
            return w.float().to(torch.bfloat16).double()
        W13 = deq(inp["w13"][e], inp["w13_scale"][e])
        W2 = deq(inp["w2"][e], inp["w2_scale"][e])
        gu = x @ W13.T
        h = torch.nn.functional.silu(gu[:, :I]) * gu[:, I:]
        h = h.float().to(torch.bfloat16).double()
        return (h @ W2.T).numpy()
    if scheme == "w4a8":
        x = torch.from_numpy(inp["x"][rows].astype(np.float64)) * \
            torch.from_numpy(inp["x_scale"][rows].astype(np.float64))[:, None]

        def deq4(codes, s):
            b = torch.from_numpy(codes.astype(np.int16))
            lo = (b & 15) - 16 * ((b & 15) >= 8).to(torch.int16)
            hi = (b >> 4) - 16 * ((b >> 4) >= 8).to(torch.int16)
            q = torch.stack([lo, hi], -1).reshape(codes.shape[0], -1).double()
            return q * torch.from_numpy(s.astype(np.float64)).repeat_interleave(32, 1)
        gu = x @ deq4(inp["w13"][e], inp["w13_scale"][e]).T
        h = torch.nn.functional.silu(gu[:, :I]) * gu[:, I:]
        s = h.abs().amax(1, keepdim=True) / 127
        hq = torch.clamp(torch.round(h / s), -127, 127) * s
        return (hq @ deq4(inp["w2"][e], inp["w2_scale"][e]).T).numpy()
    if scheme == "w8a8":
        x = torch.from_numpy(inp["x"][rows].astype(np.float64)) * \
            torch.from_numpy(inp["x_scale"][rows].astype(np.float64))[:, None]
        W13 = torch.from_numpy(inp["w13"][e].astype(np.float64)) * \
            torch.from_numpy(inp["w13_scale"][e].astype(np.float64))[:, None]
        W2 = torch.from_numpy(inp["w2"][e].astype(np.float64)) * \
            torch.from_numpy(inp["w2_scale"][e].astype(np.float64))[:, None]
        gu = x @ W13.T
        h = torch.nn.functional.silu(gu[:, :I]) * gu[:, I:]
        s = h.abs().amax(1, keepdim=True) / 127
        hq = torch.clamp(torch.round(h / s), -127, 127) * s
        return (hq @ W2.T).numpy()
    # a8w4
    xt = torch.from_numpy(inp["x"][rows]).view(torch.float8_e4m3fn).double()
    x = xt * torch.from_numpy(inp["x_scale"][rows].astype(np.float64))[:, None]
    e2m1 = {c: v for c, v in _read_table("ocp_e2m1_values.txt")}

    def deq(codes, s):
        lut = np.array([e2m1[c] for c in range(16)])
        q = np.stack([lut[codes & 15], lut[codes >> 4]], -1).reshape(codes.shape[0], -1)
        sc = torch.from_numpy(s).view(torch.float8_e8m0fnu).double().repeat_interleave(32, 1)
        return torch.from_numpy(q) * sc
    W13 = deq(inp["w13"][e], inp["w13_scale"][e])
    W2 = deq(inp["w2"][e], inp["w2_scale"][e])
    gu = x @ W13.T
    h = torch.nn.functional.silu(gu[:, :I]) * gu[:, I:]
    s = h.abs().amax(1, keepdim=True) / 448
    hq = (h / s).float().to(torch.float8_e4m3fn).double() * s
    return (hq @ W2.T).numpy()


@pytest.mark.parametrize("scheme,tol", [("w4a16", 1e-9), ("w8a8", 1e-5), ("a8w4", 1e-4),
                                        ("w4a8", 1e-5)])
def test_one_expert_top1_is_dense_ffn(scheme, tol):
    """E = 1, k = 1: the MoE layer is one dense FFN and every weight is 1."""
    sh, inp = _tiny(scheme, T=40, H=128, I=64, E=1, k=1)
    ids, w = O.route(inp["logits"], 1)
    assert np.all(ids == 0) and np.all(w == 1.0)
    r = O.moe_forward(scheme, inp["x"], inp["x_scale"], {k: inp[k] for k in
                      ("w13", "w13_scale", "w2", "w2_scale")}, ids, w)
    got = r["out32"] if scheme == "w8a8" else r["out"]
    ref = _dense_reference(scheme, inp, 0, np.arange(40))
    assert O.rel_l2(got, ref) < tol


@pytest.mark.parametrize("scheme", ["w4a16", "w8a8", "a8w4", "w4a8"])
def test_brute_force_every_expert_then_select(scheme):
    """Run every expert on every token densely, then pick each token's k
    outputs and weight them: must equal the grouped oracle."""
    sh, inp = _tiny(scheme, T=20, H=64, I=32, E=5, k=3)
    ids, w = O.route(inp["logits"], 3)
    W = {k: inp[k] for k in ("w13", "w13_scale", "w2", "w2_scale")}
    r = O.moe_forward(scheme, inp["x"], inp["x_scale"], W, ids, w)
    allY = []
    for e in range(5):
        allY.append(O.expert_ffn(scheme, inp["x"], inp["x_scale"],
                                 {k: v[e] for k, v in W.items()})["y"])
    allY = np.stack(allY)  # [E, T, H]
    T, k = ids.shape
    if scheme == "w8a8":
        acc = np.zeros((T, 64), np.float32)
        for j in range(k):
            yj = allY[ids[:, j], np.arange(T)].astype(np.float32)
            acc = (acc + (w[:, j:j + 1] * yj).astype(np.float32)).astype(np.float32)
        np.testing.assert_array_equal(r["out32"], acc)
    else:
        ref = sum(w[:, j:j + 1].astype(np.float64) * allY[ids[:, j], np.arange(T)]
                  for j in range(k))
        np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-12)


def test_w8a8_accumulators_exact_against_python_ints():
    sh, inp = _tiny("w8a8", T=6, H=96, I=32, E=2, k=1)
    ids, w = O.route(inp["logits"], 1)
    W = {k: inp[k] for k in ("w13", "w13_scale", "w2", "w2_scale")}
    r = O.moe_forward("w8a8", inp["x"], inp["x_scale"], W, ids, w, keep=("acc1", "acc2", "hq"))
    for p in range(6):
        e = int(ids[p, 0])
        for n in (0, 5, 63):
            ref = sum(int(a) * int(b) for a, b in zip(inp["x"][p], inp["w13"][e, n]))
            assert r["acc1"][p, n] == ref
        for n in (0, 17, 95):
            ref = sum(int(a) * int(b) for a, b in zip(r["hq"][p], inp["w2"][e, n]))
            assert r["acc2"][p, n] == ref


def test_a8w4_accumulators_exact_against_rationals():
    sh, inp = _tiny("a8w4", T=3, H=128, I=32, E=2, k=1)
    ids, w = O.route(inp["logits"], 1)
    W = {k: inp[k] for k in ("w13", "w13_scale", "w2", "w2_scale")}
    r = O.moe_forward("a8w4", inp["x"], inp["x_scale"], W, ids, w, keep=("acc1",))
    e2m1 = {c: Fraction(v) for c, v in _read_table("ocp_e2m1_values.txt")}
    for p in range(3):
        e = int(ids[p, 0])
        xs = torch.from_numpy(inp["x"][p]).view(torch.float8_e4m3fn).double().numpy()
        for n in (0, 33):
            codes = inp["w13"][e, n]
            q = [v for c in codes for v in (e2m1[c & 15], e2m1[c >> 4])]
            sc = [Fraction(2) ** (int(b) - 127) for b in inp["w13_scale"][e, n]]
            ref = sum(Fraction(float(xs[c])) * q[c] * sc[c // 32] for c in range(128))
            assert Fraction(float(r["acc1"][p, n])) == ref


def test_requant_rows_golden():
    for line in open(os.path.join(GOLDEN, "w8a8_requant_rows.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        hs, ss, cs = [part.split() for part in line.split("|")]
        h = np.array([[float(v) for v in hs]], np.float32)
        q, s = O.quant_rows_int8(h)
        assert abs(float(s[0]) - float(ss[0])) <= 1e-7 * max(1.0, float(ss[0]))
        np.testing.assert_array_equal(q[0], [int(v) for v in cs])


def test_requant_e4m3_row_max_maps_to_448():
    h = np.array([[3.0, -1.5, 0.75, 0.0], [0, 0, 0, 0]], np.float32)
    q, s = O.quant_rows_e4m3(h)
    assert s[0] == np.float32(3.0 / 448) and s[1] == 1.0
    np.testing.assert_array_equal(O.e4m3_values(q[0][:1]), [448.0])
    assert np.all(q[1] == 0)


def test_silu_closed_forms():
    gu = np.array([[0.0, 100.0, -100.0, 2.0, 1.0, 1.0, 1.0, 3.0]], np.float32)
    h = O.silu_mul_f32(gu, 4)
    assert h[0, 0] == 0.0
    assert h[0, 1] == 100.0
    assert h[0, 2] == 0.0
    np.testing.assert_allclose(h[0, 3], 3.0 * 2.0 / (1.0 + math.exp(-2.0)), rtol=1e-6)


def test_combine_weights_sum_to_one_reproduces_common_y():
    """If every slot of a token returns the same y, the combine returns
    y times the weight sum, which is 1 within k ulps."""
    rng = np.random.default_rng(0)
    T, k, H = 5, 4, 8
    _, w = O.route(rng.standard_normal((T, 16)).astype(np.float32), k)
    y = np.repeat(rng.standard_normal((T, 1, H)), k, 1).reshape(T * k, H)
    out = O.combine("w4a16", y, w)["out"]
    np.testing.assert_allclose(out, y.reshape(T, k, H)[:, 0], rtol=k * 2.0 ** -23)


def test_generator_shapes_and_reproducible():
    a = synth.make_inputs(W4A16_TINY)
    b = synth.make_inputs(W4A16_TINY)
    for key in a:
        if a[key] is not None:
            np.testing.assert_array_equal(a[key], b[key])
    assert a["w13"].shape == (8, 256, 128) and a["w13_scale"].shape == (8, 256, 8)
    assert a["w2"].shape == (8, 256, 64) and a["w2_scale"].shape == (8, 256, 4)
    e3 = synth.expert_weights(W4A16_TINY, 3)
    np.testing.assert_array_equal(e3["w2"], a["w2"][3])


# ---------------------------------------------------------------- comparator

def test_rel_l2_closed_forms():
    """rel_l2(a, b) = ||a - b|| / ||b|| over all elements, values worked by hand."""
    # [3, 4] against [0, 5]: difference [3, -1], ||.|| = sqrt(10); ||b|| = 5.
    assert O.rel_l2(np.array([3.0, 4.0]), np.array([0.0, 5.0])) == pytest.approx(
        math.sqrt(10) / 5, rel=1e-15)
    # orthogonal unit vectors: ||[1, -1]|| / 1
    assert O.rel_l2(np.array([1.0, 0.0]), np.array([0.0, 1.0])) == pytest.approx(
        math.sqrt(2), rel=1e-15)
    # [1, -2, 2] against [2, -2, 1]: difference [-1, 0, 1]; ||b|| = 3.
    assert O.rel_l2(np.array([1.0, -2.0, 2.0]), np.array([2.0, -2.0, 1.0])) == pytest.approx(
        math.sqrt(2) / 3, rel=1e-15)
    b = np.random.default_rng(4).standard_normal((30, 17))
    assert O.rel_l2(b, b) == 0.0
    assert O.rel_l2(np.zeros_like(b), b) == pytest.approx(1.0, rel=1e-14)
    assert O.rel_l2(3 * b, b) == pytest.approx(2.0, rel=1e-14)
    assert O.rel_l2(b * (1 + 1e-3), b) == pytest.approx(1e-3, rel=1e-9)
    # the whole array, not row by row: one bad row of 30 weighs 1/sqrt(30)
    c = b.copy()
    c[7] = -c[7]
    assert O.rel_l2(c, b) == pytest.approx(
        2 * np.linalg.norm(b[7]) / np.linalg.norm(b), rel=1e-12)


# ---------------------------------------------------------------- fp32 recipes

def _f32_rne(q: Fraction) -> Fraction:
    """Nearest IEEE binary32 value to an exact rational, ties to even
    (normal range only, which the callers assert)."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    assert -126 <= e <= 127, q
    ulp = Fraction(2) ** (e - 23)
    m = a / ulp
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * ulp


def _frac(v) -> Fraction:
    return Fraction(float(v))


def test_w8a8_rescale_rounds_twice_in_order():
    """The W8A8 rescale is f32(f32(f32(acc) * s_row) * s_col): checked against
    exact rational arithmetic rounded to fp32 after each product.  The cases
    include many where one rounding of the exact triple product, or the
    other order of the two products, gives another fp32 value."""
    rng = np.random.default_rng(12)
    n = 400
    acc = rng.integers(-2 ** 23, 2 ** 23, n)
    sx = rng.uniform(1e-3, 5e-2, n).astype(np.float32)
    sw = rng.uniform(1e-4, 1e-2, n).astype(np.float32)
    single = swapped = 0
    for i in range(n):
        got = O.rescale_w8a8(acc[i:i + 1, None], sx[i:i + 1], sw[i:i + 1])
        assert got.dtype == np.float32 and got.shape == (1, 1)
        a, x, w = Fraction(int(acc[i])), _frac(sx[i]), _frac(sw[i])
        want = _f32_rne(_f32_rne(_f32_rne(a) * x) * w)
        assert _frac(got[0, 0]) == want, (acc[i], sx[i], sw[i])
        single += _f32_rne(a * x * w) != want
        swapped += _f32_rne(_f32_rne(a * w) * x) != want
    assert single >= 20 and swapped >= 20, (single, swapped)


def test_w8a8_layer_intermediates_against_rationals():
    """gu and y of the W8A8 expert from Python integers and rationals: the
    accumulators exact, then the two-step fp32 rescale of each."""
    sh, inp = _tiny("w8a8", T=5, H=64, I=32, E=2, k=1, seed=21)
    ids, w = O.route(inp["logits"], 1)
    W = {k: inp[k] for k in ("w13", "w13_scale", "w2", "w2_scale")}
    r = O.moe_forward("w8a8", inp["x"], inp["x_scale"], W, ids, w,
                      keep=("gu", "hq", "h_scale", "acc2"))
    for p in range(5):
        e = int(ids[p, 0])
        for n in (0, 9, 40, 63):
            acc = sum(int(a) * int(b) for a, b in zip(inp["x"][p], inp["w13"][e, n]))
            want = _f32_rne(_f32_rne(Fraction(acc) * _frac(inp["x_scale"][p]))
                            * _frac(inp["w13_scale"][e, n]))
            assert _frac(r["gu"][p, n]) == want
        for n in (0, 31, 63):
            acc = sum(int(a) * int(b) for a, b in zip(r["hq"][p], inp["w2"][e, n]))
            assert r["acc2"][p, n] == acc
            want = _f32_rne(_f32_rne(Fraction(acc) * _frac(r["h_scale"][p]))
                            * _frac(inp["w2_scale"][e, n]))
            assert _frac(r["y_pairs"][p, n]) == want


def _tie_rows(qmax, n_rows, seed, midpoints):
    """Rows [qmax * s, h] whose quotient h / s is exactly a midpoint m
    between two codes, with s an fp32 of 16 significant bits (so h = m * s
    and qmax * s are exact fp32 values and f32(qmax * s / qmax) = s).
    Returns (h, s, m) triples where RN(h * RN(1/s)) is not m: there the
    correctly rounded quotient and the reciprocal product take different
    sides of the tie."""
    rng = np.random.default_rng(seed)
    rows = []
    tries = 0
    while len(rows) < n_rows:
        tries += 1
        assert tries < 200000
        mant = int(rng.integers(2 ** 15, 2 ** 16))
        s = Fraction(mant, 2 ** 15) * Fraction(2) ** int(rng.integers(-8, 4))
        m = midpoints[int(rng.integers(0, len(midpoints)))] * (1 if rng.integers(0, 2) else -1)
        h = m * s
        assert _f32_rne(h) == h and _f32_rne(qmax * s) == qmax * s
        if _f32_rne(_f32_rne(h) * _f32_rne(1 / s)) != m:
            rows.append((h, s, m))
    return rows


def test_requant_int8_quotient_is_correctly_rounded():
    """Per-row int8 requantization: code = round_half_even(f32(h / s)) with
    the correctly rounded fp32 quotient.  Every row here puts h / s exactly
    on a .5 tie where h * RN(1/s) lands off the tie, so a reciprocal-product
    quotient would give the other code."""
    mids = [Fraction(2 * n + 1, 2) for n in range(0, 126)]
    rows = _tie_rows(127, 40, 31, mids)
    h = np.array([[float(127 * s), float(hv)] for hv, s, _ in rows], np.float32)
    q, sc = O.quant_rows_int8(h)
    for i, (hv, s, m) in enumerate(rows):
        assert _frac(sc[i]) == s
        fl = m.numerator // m.denominator  # floor
        even = fl if fl % 2 == 0 else fl + 1
        assert q[i, 0] == 127 and q[i, 1] == even, (float(hv), float(s), m)


def test_requant_e4m3_quotient_is_correctly_rounded():
    """Per-row e4m3 requantization: code = RNE(f32(h / s)) with the correctly
    rounded fp32 quotient; h / s sits exactly halfway between two e4m3
    values, where h * RN(1/s) lands off the tie.  Expected codes from torch's
    own float8_e4m3fn cast of the exact quotient."""
    vals = np.sort(np.unique(np.abs(O.E4M3_TABLE[~np.isnan(O.E4M3_TABLE)])))
    normal = vals[vals >= 2.0 ** -6]
    mids = [Fraction(float(a)) / 2 + Fraction(float(b)) / 2 for a, b in zip(normal[:-1], normal[1:])]
    rows = _tie_rows(448, 40, 32, mids)
    h = np.array([[float(448 * s), float(hv)] for hv, s, _ in rows], np.float32)
    q, sc = O.quant_rows_e4m3(h)
    want = torch.tensor([float(m) for _, _, m in rows], dtype=torch.float32) \
        .to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for i, (hv, s, m) in enumerate(rows):
        assert _frac(sc[i]) == s
        assert q[i, 0] == 0x7E and q[i, 1] == want[i], (float(hv), float(s), m)


# ---------------------------------------------------------------- W4A8

def test_w4a8_group_sums_against_python_ints():
    """Each 32-wide group's int8 x int4 dot product, against Python integers
    (two's-complement nibbles read by hand, low nibble = even K)."""
    sh, inp = _tiny("w4a8", T=4, H=128, I=32, E=2, k=1, seed=41)
    acc = O.group_sums_int4(inp["x"], inp["w13"][1])
    assert acc.shape == (4, 64, 4) and acc.dtype == np.int64

    def nib(v):
        return v - 16 if v >= 8 else v
    for p in range(4):
        for n in (0, 17, 63):
            row = inp["w13"][1, n]
            q = [nib(int(b) & 15) if c % 2 == 0 else nib(int(b) >> 4)
                 for b in row for c in (0, 1)]
            for g in range(4):
                want = sum(int(inp["x"][p, c]) * q[c] for c in range(32 * g, 32 * g + 32))
                assert acc[p, n, g] == want


def test_w4a8_group_scales_against_rationals():
    """The group scales multiply the exact integer group sums, then the row
    scale: one fp64 rounding of the exact rational value."""
    rng = np.random.default_rng(42)
    acc = rng.integers(-32512, 32513, (3, 5, 16))
    sc = rng.uniform(0.005, 0.02, (5, 16)).astype(np.float16)
    sr = rng.uniform(1e-3, 5e-2, 3).astype(np.float32)
    got = O.apply_group_scales(acc, sc, sr)
    for p in range(3):
        for n in range(5):
            exact = Fraction(float(sr[p])) * sum(Fraction(float(sc[n, g])) * int(acc[p, n, g])
                                                 for g in range(16))
            assert got[p, n] == float(exact)  # Python's int/int division rounds correctly


def test_w4a8_unit_scales_reduce_to_the_integer_dot_product():
    """With every group scale 1 and a unit token scale, gu is the plain
    integer dot product of the int8 row with the int4 row (exact in fp32
    below 2^24)."""
    sh, inp = _tiny("w4a8", T=6, H=256, I=64, E=1, k=1, seed=43)
    s13 = np.ones_like(inp["w13_scale"][0])
    r = O.expert_w4a8(inp["x"], np.ones(6, np.float32), inp["w13"][0], s13, inp["w2"][0],
                      np.ones_like(inp["w2_scale"][0]))
    q = O.int4_values(inp["w13"][0]).astype(np.int64)
    dot = inp["x"].astype(np.int64) @ q.T
    np.testing.assert_array_equal(r["gu"], dot.astype(np.float32))
    np.testing.assert_array_equal(r["acc1"].sum(axis=2), dot)
