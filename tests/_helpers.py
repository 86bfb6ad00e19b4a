"""Shared test helpers: moving generator outputs to the GPU and running the
oracle on all tokens or on a sample of tokens."""
import numpy as np
import torch

import oracle as O
from quantized_mixture_experts_moe_amd import synth

WEIGHT_KEYS = ("w13", "w13_scale", "w2", "w2_scale")


def to_gpu(a, dev="cuda"):
    if a is None:
        return None
    if a.dtype == np.uint16:  # bf16 bits
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def gpu_inputs(inp, dev="cuda"):
    return {k: to_gpu(v, dev) for k, v in inp.items()}


def bf16_to_np(t):
    """bf16 tensor -> float64 numpy (exact)."""
    return t.float().cpu().numpy().astype(np.float64)


def oracle_tokens(shape, inp, tokens, weights=None, keep=()):
    """Oracle output rows for the given token indices (routing from logits)."""
    tokens = np.asarray(tokens)
    ids, w = O.route(inp["logits"][tokens], shape.topk)
    xs = None if inp["x_scale"] is None else inp["x_scale"][tokens]
    if weights is None:
        cache = {}

        def weights(e):
            if e not in cache:
                cache[e] = synth.expert_weights(shape, e)
            return cache[e]
    r = O.moe_forward(shape.scheme, inp["x"][tokens], xs, weights, ids, w, keep=keep)
    r["topk_ids"], r["topk_w"] = ids, w
    return r
