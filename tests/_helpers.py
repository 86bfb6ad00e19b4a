"""Shared test helpers: moving generator outputs to the GPU, running the
oracle over every token (experts on a thread pool), and recording parity
margins."""
import json
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle as O

WEIGHT_KEYS = ("w13", "w13_scale", "w2", "w2_scale")
TOL = {"w4a16": 5e-3, "a8w4": 5e-3, "w8a8": 1e-5, "w4a8": 5e-3}

# (case, quantity, value, tolerance) of every fp comparison, in test order;
# conftest writes them to $QMOE_MARGINS_OUT at the end of the session.
MARGINS = []


def record_margin(case: str, quantity: str, value: float, tol: float):
    MARGINS.append({"case": case, "quantity": quantity, "rel_l2": float(value),
                    "tol": float(tol), "share_of_tol": float(value) / float(tol)})
    print(f"  {case} {quantity} rel_l2 {value:.3e} ({100 * value / tol:.1f}% of {tol:g})",
          flush=True)


def write_margins():
    path = os.environ.get("QMOE_MARGINS_OUT")
    if path and MARGINS:
        with open(path, "a") as f:
            for m in MARGINS:
                f.write(json.dumps(m) + "\n")


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


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n) // 2)


def oracle_full(scheme, inp, ids, w, keep=()):
    """The oracle over every (token, slot) pair, the experts spread over a
    thread pool (two BLAS threads each); the weights are the stacked arrays
    of ``inp``."""
    from threadpoolctl import threadpool_limits

    W = {k: inp[k] for k in WEIGHT_KEYS}
    with threadpool_limits(2), ThreadPoolExecutor(_workers()) as ex:
        return O.moe_forward(scheme, inp["x"], inp["x_scale"], W, ids, w, keep=keep,
                             map_fn=ex.map)
