"""Workload shapes of the grouped, weight-quantized MoE FFN.

Each shape names a quantization scheme and the sizes T (tokens), H (hidden),
I (expert intermediate), E (experts) and k (experts per token).  The schemes
are the three lowerings the pages discuss:

* ``w4a16`` -- symmetric int4 weights with one fp16 scale per 32 values along
  K, bf16 activations; the pages' "dequantise-then-bf16-dot" lowering
  (vLLM issue "Evaluate native IU4/IU8 WMMA for grouped-INT MoE prefill on
  gfx1151", section Constraint; hip-ep PR "perf(qmoe): group prefill expert
  matmuls", description: symmetric int4 expert projections).
* ``w8a8`` -- int8 per-output-channel weights and int8 per-token activations,
  int32 accumulation (same issue, sections Constraint and Scope).
* ``a8w4`` -- fp8 e4m3 activations with a per-token scale and MXFP4 (e2m1
  with one e8m0 scale per 32 along K) weights (aiter PR 6090, sections
  Motivation and Changes: model_dim 4096, 512 experts, topk 10, fp8 act,
  MXFP4 weight, inter_dim 1024).
* ``w4a8`` -- the int4 group-32 weights of w4a16 with the int8 per-token
  activations of w8a8, upconverted to 8 bits for an integer product (vLLM
  issue, section Constraint: W4A8 with upconversion of weights to IU8
  before the MMA).
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional

SCHEMES = ("w4a16", "w8a8", "a8w4", "w4a8")
# Numeric codes shared with the C ABI (qmoe_scheme in include/qmoe.h).
SCHEME_CODE = {"w4a16": 0, "w8a8": 1, "a8w4": 2, "w4a8": 3}


@dataclass(frozen=True)
class MoEShape:
    name: str
    scheme: str
    tokens: int
    hidden: int
    inter: int
    experts: int
    topk: int
    seed: int
    # Token rows drawn by the generator; a smaller ``tokens`` takes the
    # leading rows so that a token sweep shares weights and activations.
    tokens_drawn: int = 0
    # Router-logit bias: Zipf exponent over expert rank (None = no bias).
    zipf_s: Optional[float] = None

    def __post_init__(self):
        assert self.scheme in SCHEMES
        if self.tokens_drawn == 0:
            object.__setattr__(self, "tokens_drawn", self.tokens)
        assert self.tokens <= self.tokens_drawn

    @property
    def pairs(self) -> int:
        return self.tokens * self.topk

    def with_tokens(self, tokens: int) -> "MoEShape":
        assert tokens <= self.tokens_drawn
        return replace(self, tokens=tokens, name=f"{self.name.split('@')[0]}@T{tokens}")

    def useful_flops(self) -> float:
        """2 flops per multiply-add of the three projections, pairs only."""
        return 6.0 * self.hidden * self.inter * self.pairs


# Small shape the oracle finishes in well under a second.
W4A16_TINY = MoEShape("w4a16_tiny", "w4a16", tokens=64, hidden=256, inter=128,
                      experts=8, topk=2, seed=1000)
# Qwen3-MoE-style expert block at a 128-token prefill.
W4A16_QWEN3MOE = MoEShape("w4a16_qwen3moe_t128", "w4a16", tokens=128, hidden=2048,
                          inter=768, experts=128, topk=8, seed=1001)
# Same block, int8 weights and per-token int8 activations, 2048 tokens.
W8A8_T2048 = MoEShape("w8a8_t2048", "w8a8", tokens=2048, hidden=2048, inter=768,
                      experts=128, topk=8, seed=1002)
# fp8 x MXFP4 large MoE (hidden 4096, 512 experts, top-10, inter 1024) at
# 4096 tokens; the sweep takes 256, 1024, 4096 and 8192 leading tokens.
A8W4_LARGE = MoEShape("a8w4_large@T4096", "a8w4", tokens=4096, hidden=4096, inter=1024,
                      experts=512, topk=10, seed=1003, tokens_drawn=8192)
A8W4_SWEEP_TOKENS = (256, 1024, 4096, 8192)
# The same block split over two or four GPUs by tensor parallelism: each
# GPU holds every expert with a share of the intermediate (inter 512, 256;
# aiter PR 6090, section Changes).  Stage 1 is then column-parallel and
# stage 2 row-parallel; one GPU's share is exactly this shape.
A8W4_TP2 = MoEShape("a8w4_tp2@T4096", "a8w4", tokens=4096, hidden=4096, inter=512,
                    experts=512, topk=10, seed=1005, tokens_drawn=8192)
A8W4_TP4 = MoEShape("a8w4_tp4@T4096", "a8w4", tokens=4096, hidden=4096, inter=256,
                    experts=512, topk=10, seed=1006, tokens_drawn=8192)
# Long prefill with a Zipf-skewed router: a few experts get most rows.
W4A16_SKEWED = MoEShape("w4a16_skewed_t8192", "w4a16", tokens=8192, hidden=4096,
                        inter=1024, experts=512, topk=10, seed=1004, zipf_s=1.2)

# W4A8 on the Qwen3-MoE-style block (128 and 2048 tokens) and on the skewed
# long prefill.
W4A8_QWEN3MOE = MoEShape("w4a8_qwen3moe_t128", "w4a8", tokens=128, hidden=2048, inter=768,
                         experts=128, topk=8, seed=1007, tokens_drawn=2048)
W4A8_T2048 = MoEShape("w4a8_t2048", "w4a8", tokens=2048, hidden=2048, inter=768, experts=128,
                      topk=8, seed=1007)
W4A8_SKEWED = MoEShape("w4a8_skewed_t8192", "w4a8", tokens=8192, hidden=4096, inter=1024,
                       experts=512, topk=10, seed=1008, zipf_s=1.2)

ALL_SHAPES = {s.name: s for s in (W4A16_TINY, W4A16_QWEN3MOE, W8A8_T2048, A8W4_LARGE,
                                  A8W4_TP2, A8W4_TP4, W4A16_SKEWED, W4A8_QWEN3MOE, W4A8_T2048,
                                  W4A8_SKEWED)}


def shape_by_name(name: str) -> MoEShape:
    if name in ALL_SHAPES:
        return ALL_SHAPES[name]
    base, _, t = name.partition("@T")
    for s in ALL_SHAPES.values():
        if s.name.split("@")[0] == base:
            return s.with_tokens(int(t)) if t else s
    raise KeyError(name)


def default_block_m(shape: MoEShape) -> int:
    """Tile height for a shape: the library's qmoe_default_block_m, i.e. the
    gfx950 tile table's entry for the shape and token bucket (a sweep with a
    bit-exact accuracy gate, ``bench.py --tile-sweep``), else its rule on the
    mean rows per expert."""
    from . import ops  # the library binding (loaded lazily: ops imports this module)

    bm = int(ops.lib().qmoe_default_block_m(SCHEME_CODE[shape.scheme], shape.tokens,
                                            shape.hidden, shape.inter, shape.experts,
                                            shape.topk))
    if bm == 0:
        raise ValueError(f"no tile height for {shape}")
    return bm
