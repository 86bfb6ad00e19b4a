"""GPU: the place of a K step's weight loads in the 128-row stage-1 tiles of
8 waves (in front of the step's MFMAs, or behind them; QMOE_TILE s1lb)
changes only when the loads are issued, never what is summed: every output
must be the same bits either way.  Shapes on both sides of the rule (48 pairs
per expert), both weight layouts, the three schemes whose stage 1 takes
8-wave blocks at 128 rows, K loops of four and of eight steps.
"""
import pytest
import torch

from quantized_mixture_experts_moe_amd import ops, synth
from quantized_mixture_experts_moe_amd.shapes import MoEShape

from _helpers import WEIGHT_KEYS, gpu_inputs

pytestmark = pytest.mark.gpu


def _run(sh, inp, prepacked, tile, monkeypatch):
    monkeypatch.setenv("QMOE_TILE", tile)
    g = gpu_inputs(inp)
    W = {k: g[k] for k in WEIGHT_KEYS}
    if prepacked:
        W = ops.prepack_weights(sh.scheme, W)
    r = ops.moe_forward(sh.scheme, g["logits"], g["x"], g["x_scale"], W, sh.topk, 128)
    torch.cuda.synchronize()
    monkeypatch.delenv("QMOE_TILE")
    return r


@pytest.mark.parametrize("prepacked", [False, True], ids=["canonical", "prepacked"])
@pytest.mark.parametrize("scheme", ["a8w4", "w4a16", "w4a8"])
@pytest.mark.parametrize("T,H", [(256, 1024), (1024, 1024), (1024, 2048)])
def test_weight_load_order_gives_the_same_bits(scheme, T, H, prepacked, monkeypatch):
    sh = MoEShape(f"loadorder_{scheme}_T{T}_H{H}", scheme, tokens=T, hidden=H, inter=512,
                  experts=32, topk=4, seed=4242 + T + H)
    print(f"load order {sh.name} {'prepacked' if prepacked else 'canonical'}", flush=True)
    inp = synth.make_inputs(sh)
    front = _run(sh, inp, prepacked, "s1w=8,s1lb=0", monkeypatch)
    behind = _run(sh, inp, prepacked, "s1w=8,s1lb=1", monkeypatch)
    assert torch.equal(front["topk_ids"], behind["topk_ids"])
    assert torch.equal(front["y_pairs"].view(torch.int16), behind["y_pairs"].view(torch.int16))
    assert torch.equal(front["out"].view(torch.int16), behind["out"].view(torch.int16))
