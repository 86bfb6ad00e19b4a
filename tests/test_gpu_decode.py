"""GPU parity of qmoe_decode, the one-launch path for up to 16 tokens
(vLLM issue "Evaluate native IU4/IU8 WMMA for grouped-INT MoE prefill on
gfx1151", section Problem: decode is bound by weight streaming and dispatch
count; aiter PR 6090, section Changes: token bucket 1-256).

Every output (routing ids and weights, per-pair expert outputs, the combined
output) must equal the multi-launch path's bit for bit, and both are checked
against the CPU oracle run on its own routing.  One workspace serves every
call of a test: the kernel's arrival counters must come back to zero after
each call, and its flag word must stay clear.  The full-size decode buckets
of each scheme are covered in test_gpu_parity (test_decode_buckets_every_token).
"""
import numpy as np
import pytest
import torch

import oracle as O
from quantized_mixture_experts_moe_amd import ops, synth
from quantized_mixture_experts_moe_amd.shapes import MoEShape

from _helpers import TOL, WEIGHT_KEYS, bf16_to_np, gpu_inputs, record_margin
from test_gpu_parity import _run_decode, _run_gpu, _same_outputs

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(msg, flush=True)


def _oracle_check(case, sh, inp, d):
    ids_o, w_o = O.route(inp["logits"], sh.topk)
    np.testing.assert_array_equal(d["topk_ids"].cpu().numpy(), ids_o)
    np.testing.assert_allclose(d["topk_w"].cpu().numpy(), w_o, rtol=2.0 ** -23, atol=0)
    ref = O.moe_forward(sh.scheme, inp["x"], inp["x_scale"], {k: inp[k] for k in WEIGHT_KEYS},
                        ids_o, w_o)
    if sh.scheme == "w8a8":
        np.testing.assert_array_equal(d["y_pairs"].cpu().numpy(), ref["y_pairs"])
        err = O.rel_l2(d["out_f32"].cpu().numpy(), ref["out32"])
        record_margin(case, "out_f32", err, TOL["w8a8"])
        assert err <= TOL["w8a8"]
    else:
        ey = O.rel_l2(bf16_to_np(d["y_pairs"]), ref["y_pairs"])
        eo = O.rel_l2(bf16_to_np(d["out"]), ref["out"])
        record_margin(case, "y_pairs", ey, TOL[sh.scheme])
        record_margin(case, "out", eo, TOL[sh.scheme])
        assert ey <= TOL[sh.scheme] and eo <= TOL[sh.scheme]


def _shape(scheme, T, E, k, H=512, I=256, seed=77):
    return MoEShape(f"decode_{scheme}_T{T}_E{E}_k{k}", scheme, tokens=T, hidden=H, inter=I,
                    experts=E, topk=k, seed=seed)


LAYOUTS = pytest.mark.parametrize("prepacked", [False, True], ids=["canonical", "prepacked"])
SCHEMES = pytest.mark.parametrize("scheme", ["w4a16", "w8a8", "a8w4", "w4a8"])


@SCHEMES
@LAYOUTS
def test_decode_token_counts_share_one_workspace(scheme, prepacked):
    """T = 16, 1, 5, 16 in a row on one workspace: each call equals the
    multi-launch path and the oracle."""
    ws = None
    for T in (16, 1, 5, 16):
        sh = _shape(scheme, T, E=64, k=6, seed=70 + T)
        case = f"{sh.name} {'prepacked' if prepacked else 'canonical'}"
        _flush(f"decode {case}")
        inp = synth.make_inputs(sh)
        d = _run_decode(sh, inp, prepacked, ws=ws)
        ws = d["ws"]
        assert ops.check_flags(ws) == 0
        r = _run_gpu(sh, inp, 16, 0, prepacked)
        _same_outputs(d, r, scheme)
        _oracle_check(case, sh, inp, d)


@SCHEMES
@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (3, 4, 4), (16, 16, 16), (16, 1024, 16),
                                   (7, 300, 5), (2, 256, 2)])
def test_decode_routing_extremes(scheme, T, E, k):
    """One expert; every expert taken by every token; the largest pair count
    (256) with 16 rows in a slot; 1024 experts (16 logits per lane);
    an expert count that is not a multiple of 64."""
    sh = _shape(scheme, T, E, k, seed=300 + T + E + k)
    case = f"{sh.name} prepacked"
    _flush(f"decode {case}")
    inp = synth.make_inputs(sh)
    d = _run_decode(sh, inp, True)
    assert ops.check_flags(d["ws"]) == 0
    r = _run_gpu(sh, inp, 16, 0, True)
    _same_outputs(d, r, scheme)
    _oracle_check(case, sh, inp, d)


@SCHEMES
def test_decode_all_tokens_on_the_same_experts(scheme):
    """Every token routes to the same k experts: each touched expert's slot
    holds all 16 rows (the requantization of a slot's rows by its last
    stage-1 unit covers 16 rows).  Outputs equal the multi-launch path's bit
    for bit; against the oracle the routing is exact and y_pairs within the
    tolerance.  The combined output's relative L2 is recorded, not asserted:
    with 64 pairs on four experts one fp8 code of the requantized h that
    lands on the other side of a rounding tie (an ulp-level difference of h,
    from the hardware exp2 and reciprocal of the SiLU, at the top of the
    e4m3 range where a step is 1/14 of the row's absmax) moves that pair's
    row by about 2% (measured for a8w4 on this input: one pair at 2.2e-2,
    the other 63 at the bf16 floor of 1.6e-3), and the combined output of
    its token follows; over a routed batch such flips average out (the
    decode buckets and the other tests assert the output)."""
    sh = _shape(scheme, 16, 32, 4, seed=901)
    inp = synth.make_inputs(sh)
    logits = np.full((16, 32), -4.0, np.float32)
    logits[:, [3, 9, 17, 30]] = np.array([2.0, 1.5, 1.0, 0.5], np.float32) + \
        np.linspace(0, 0.25, 16, dtype=np.float32)[:, None]
    inp["logits"] = logits
    d = _run_decode(sh, inp, True)
    assert ops.check_flags(d["ws"]) == 0
    assert set(np.unique(d["topk_ids"].cpu().numpy()).tolist()) == {3, 9, 17, 30}
    r = _run_gpu(sh, inp, 16, 0, True)
    _same_outputs(d, r, scheme)
    ids_o, w_o = O.route(inp["logits"], sh.topk)
    np.testing.assert_array_equal(d["topk_ids"].cpu().numpy(), ids_o)
    np.testing.assert_allclose(d["topk_w"].cpu().numpy(), w_o, rtol=2.0 ** -23, atol=0)
    ref = O.moe_forward(sh.scheme, inp["x"], inp["x_scale"], {k: inp[k] for k in WEIGHT_KEYS},
                        ids_o, w_o)
    case = f"{sh.name} same experts"
    if scheme == "w8a8":
        np.testing.assert_array_equal(d["y_pairs"].cpu().numpy(), ref["y_pairs"])
        record_margin(case, "out_f32 (not asserted)",
                      O.rel_l2(d["out_f32"].cpu().numpy(), ref["out32"]), TOL[scheme])
    else:
        ey = O.rel_l2(bf16_to_np(d["y_pairs"]), ref["y_pairs"])
        record_margin(case, "y_pairs", ey, TOL[scheme])
        assert ey <= TOL[scheme]
        record_margin(case, "out (not asserted)", O.rel_l2(bf16_to_np(d["out"]), ref["out"]),
                      TOL[scheme])


@SCHEMES
def test_decode_long_rows(scheme):
    """Hidden 2048 and intermediate 1536: stage-1 K loops of 8-16 steps and
    stage-2 K loops longer than the prefetch ring."""
    sh = _shape(scheme, 4, 32, 4, H=2048, I=1536, seed=505)
    inp = synth.make_inputs(sh)
    d = _run_decode(sh, inp, True)
    assert ops.check_flags(d["ws"]) == 0
    r = _run_gpu(sh, inp, 16, 0, True)
    _same_outputs(d, r, scheme)
    _oracle_check(f"{sh.name} long rows", sh, inp, d)


@pytest.mark.parametrize("var,val", [("QMOE_DECODE_RING", "4"), ("QMOE_DECODE_RING", "6"),
                                     ("QMOE_DECODE_G", "1"), ("QMOE_DECODE_G", "2"),
                                     ("QMOE_DECODE_G", "4"), ("QMOE_DECODE_G", "8")])
@pytest.mark.parametrize("scheme", ["a8w4", "w8a8"])
def test_decode_work_split_gives_the_same_bits(scheme, var, val, monkeypatch):
    """QMOE_DECODE_RING (how far ahead the K loops load) and QMOE_DECODE_G
    (32-column chunks per stage-2 unit) change only how the work is split."""
    sh = _shape(scheme, 8, 64, 8, H=1024, I=512, seed=606)
    inp = synth.make_inputs(sh)
    monkeypatch.setenv(var, val)
    d = _run_decode(sh, inp, True)
    monkeypatch.delenv(var)
    assert ops.check_flags(d["ws"]) == 0
    r = _run_gpu(sh, inp, 16, 0, True)
    _same_outputs(d, r, scheme)


@pytest.mark.parametrize("scheme", ["w8a8", "a8w4", "w4a16", "w4a8"])
@pytest.mark.parametrize("H,ring", [(768, "4"), (1280, "4"), (1024, "6"), (1536, "6")])
def test_decode_k_loop_tails_with_four_row_slots(scheme, H, ring, monkeypatch):
    """K loops whose last steps are loaded conditionally (steps not a
    multiple of the prefetch depth), with slots of four to six rows: the
    fourth row's accumulator is the last register of an MFMA result and the
    first one copied out at the loop's exit.  (Without wait states added
    after the MFMAs there, W8A8 lost the last K step of that row.)"""
    if scheme == "a8w4" and H % 256:
        pytest.skip("a8w4 needs H % 256 == 0")
    sh = _shape(scheme, 16, 64, 8, H=H, I=512, seed=622)
    inp = synth.make_inputs(sh)
    monkeypatch.setenv("QMOE_DECODE_RING", ring)
    d = _run_decode(sh, inp, True)
    monkeypatch.delenv("QMOE_DECODE_RING")
    assert ops.check_flags(d["ws"]) == 0
    r = _run_gpu(sh, inp, 16, 0, True)
    _same_outputs(d, r, scheme)


def test_decode_repeat_is_deterministic():
    sh = _shape("a8w4", 16, 128, 8, H=1024, I=512, seed=808)
    inp = synth.make_inputs(sh)
    g = gpu_inputs(inp)
    W = ops.prepack_weights("a8w4", {k: g[k] for k in WEIGHT_KEYS})
    first = ops.decode_forward("a8w4", g["logits"], g["x"], g["x_scale"], W, sh.topk)
    ws = first["ws"]
    outs = [first["out"].clone()]
    for _ in range(20):
        outs.append(ops.decode_forward("a8w4", g["logits"], g["x"], g["x_scale"], W, sh.topk,
                                       ws=ws)["out"].clone())
    torch.cuda.synchronize()
    assert ops.check_flags(ws) == 0
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
