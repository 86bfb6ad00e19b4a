"""Seeded synthetic inputs for the grouped MoE FFN.

This module only draws random numbers and stores them in the canonical
formats the library reads; it holds none of the MoE arithmetic (routing,
grouping, the projections, the epilogue or the combine).  Both the CPU oracle
(through the tests) and the GPU path read exactly these bytes.

Canonical layouts (row-major, K contiguous):

* ``logits``  fp32 ``[T, E]``: N(0,1), plus ``log p(r)`` with
  ``p(r) ~ r^-s`` over expert rank ``r = e + 1`` when a Zipf bias is set.
* ``x``: w4a16 -> bf16 bits (uint16) ``[T, H]`` from N(0,1);
  w8a8 and w4a8 -> int8 ``[T, H]`` + fp32 ``x_scale [T]``; a8w4 -> OCP e4m3 codes
  (uint8) ``[T, H]`` + fp32 ``x_scale [T]``.  The quantized activations come
  from the same bf16 N(0,1) source, quantized per token as
  ``s = absmax / qmax`` (qmax 127 or 448), round-half-even, saturating.
* ``w13`` ``[E, 2I, H]`` (rows 0..I-1 gate, I..2I-1 up) and ``w2 [E, H, I]``:
  w4a16 and w4a8 -> two's-complement int4 packed two per byte, low nibble =
  even K (uniform bytes = independent uniform codes in [-8, 7]), fp16
  scales ``[E, N, K/32]`` uniform in [0.005, 0.02];
  w8a8 -> int8 per output channel from N(0, 1/K) masters, fp32 scales ``[E, N]``;
  a8w4 -> e2m1 codes packed the same way (uniform over the 16 codes), e8m0
  scale bytes ``[E, N, K/32]`` uniform over {120, 121, 122} (2^-7..2^-5).

Every tensor comes from its own counter-style stream
``numpy.random.default_rng([seed, stream, index])`` so one expert's weights
can be regenerated without drawing the others.
"""
from __future__ import annotations

import numpy as np
import torch

from .shapes import MoEShape

_S_LOGITS, _S_X = 1, 2
_S_W13, _S_W13S, _S_W2, _S_W2S = 10, 11, 12, 13


def _rng(shape: MoEShape, stream: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng([shape.seed, stream, index])


def _random_bytes(rng: np.random.Generator, n: int) -> np.ndarray:
    words = rng.integers(0, np.iinfo(np.uint64).max, size=(n + 7) // 8, dtype=np.uint64,
                         endpoint=True)
    return words.view(np.uint8)[:n]


def _bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def logits(shape: MoEShape) -> np.ndarray:
    z = _rng(shape, _S_LOGITS).standard_normal((shape.tokens_drawn, shape.experts),
                                               dtype=np.float32)
    if shape.zipf_s is not None:
        r = np.arange(1, shape.experts + 1, dtype=np.float64)
        p = r ** (-shape.zipf_s)
        bias = np.log(p / p.sum())
        z = (z.astype(np.float64) + bias[None, :]).astype(np.float32)
    return np.ascontiguousarray(z[: shape.tokens])


def activations(shape: MoEShape):
    """Return (x, x_scale); x_scale is None for w4a16."""
    src = _rng(shape, _S_X).standard_normal((shape.tokens_drawn, shape.hidden),
                                            dtype=np.float32)[: shape.tokens]
    bits = _bf16_bits_from_f32(src)
    if shape.scheme == "w4a16":
        return bits, None
    xf = torch.from_numpy(_bf16_bits_to_f32(bits))
    int8 = shape.scheme in ("w8a8", "w4a8")
    qmax = 127.0 if int8 else 448.0
    amax = xf.abs().amax(dim=1)
    s = torch.where(amax > 0, amax / qmax, torch.ones_like(amax))
    v = xf / s[:, None]
    if int8:
        q = torch.clamp(torch.round(v), -127, 127).to(torch.int8).numpy()
    else:
        v = torch.clamp(v, -448.0, 448.0)
        q = v.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return np.ascontiguousarray(q), s.numpy().astype(np.float32)


def _packed_codes(shape: MoEShape, stream: int, e: int, n: int, kdim: int) -> np.ndarray:
    return _random_bytes(_rng(shape, stream, e), n * kdim // 2).reshape(n, kdim // 2)


def _group_scales(shape: MoEShape, stream: int, e: int, n: int, kdim: int) -> np.ndarray:
    rng = _rng(shape, stream, e)
    if shape.scheme in ("w4a16", "w4a8"):
        return rng.uniform(0.005, 0.02, size=(n, kdim // 32)).astype(np.float16)
    return rng.integers(120, 123, size=(n, kdim // 32), dtype=np.uint8)  # a8w4 e8m0


def _int8_channel(shape: MoEShape, stream: int, e: int, n: int, kdim: int):
    w = _rng(shape, stream, e).standard_normal((n, kdim), dtype=np.float32)
    w *= np.float32(1.0 / np.sqrt(kdim))
    wt = torch.from_numpy(w)
    amax = wt.abs().amax(dim=1)
    s = torch.where(amax > 0, amax / 127.0, torch.ones_like(amax))
    q = torch.clamp(torch.round(wt / s[:, None]), -127, 127).to(torch.int8)
    return q.numpy(), s.numpy().astype(np.float32)


def expert_weights(shape: MoEShape, e: int) -> dict:
    """Weights of expert ``e`` alone: w13, w13_scale, w2, w2_scale."""
    H, I = shape.hidden, shape.inter
    if shape.scheme == "w8a8":
        w13, s13 = _int8_channel(shape, _S_W13, e, 2 * I, H)
        w2, s2 = _int8_channel(shape, _S_W2, e, H, I)
    else:
        w13 = _packed_codes(shape, _S_W13, e, 2 * I, H)
        s13 = _group_scales(shape, _S_W13S, e, 2 * I, H)
        w2 = _packed_codes(shape, _S_W2, e, H, I)
        s2 = _group_scales(shape, _S_W2S, e, H, I)
    return {"w13": w13, "w13_scale": s13, "w2": w2, "w2_scale": s2}


def all_weights(shape: MoEShape) -> dict:
    """Stacked weights of every expert, ``[E, ...]`` per tensor."""
    first = expert_weights(shape, 0)
    out = {k: np.empty((shape.experts,) + v.shape, v.dtype) for k, v in first.items()}
    for key, v in first.items():
        out[key][0] = v
    for e in range(1, shape.experts):
        for key, v in expert_weights(shape, e).items():
            out[key][e] = v
    return out


def make_inputs(shape: MoEShape, with_weights: bool = True) -> dict:
    x, xs = activations(shape)
    d = {"logits": logits(shape), "x": x, "x_scale": xs}
    if with_weights:
        d.update(all_weights(shape))
    return d
