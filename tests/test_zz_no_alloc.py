"""qmoe_align_noalloc (the align entry point whose workspace is a device
array inside the library, for callers that cannot allocate) against
qmoe_align on the same ids: every output bit for bit, and the flag word, on
two calls in a row, the second smaller, through each of the align paths."""
import numpy as np
import pytest
import torch

import oracle as O
from quantized_mixture_experts_moe_amd import ops

from _helpers import to_gpu

pytestmark = pytest.mark.gpu

KEYS = ("sorted_pair_ids", "tile_expert", "expert_offsets", "num_padded")


def _ids(T, E, k, seed, bad=None):
    rng = np.random.default_rng(seed)
    ids, _ = O.route(rng.standard_normal((T, E)).astype(np.float32), k)
    if bad is not None:
        ids[bad] = E + 3  # out of range: dropped and flagged (bit 0)
    return ids


def _compare(ids_np, E, bm):
    ids = to_gpu(ids_np)
    ref = ops.align(ids, E, bm)
    flags = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    got = ops.align_noalloc(ids, E, bm, flags=flags)
    torch.cuda.synchronize()
    for key in KEYS:
        assert torch.equal(got[key], ref[key]), key
    assert int(flags.item()) == ops.check_flags(ref["ws"])
    return int(flags.item())


# (first call, second call): the second has fewer tokens, so stale counts,
# chunk flags and totals of the first call sit in the shared array when it
# runs.  One block up to 512 tokens, two launches up to 16384, three beyond.
CASES = [
    ((3000, 64, 4, 64), (700, 64, 4, 32)),
    ((16384, 1024, 10, 128), (4096, 512, 10, 128)),
    ((40000, 128, 8, 64), (20000, 64, 2, 16)),
    ((512, 512, 10, 16), (1, 512, 10, 16)),
]


@pytest.mark.parametrize("first,second", CASES)
def test_align_noalloc_matches_align(first, second):
    print(f"align_noalloc {first} then {second}", flush=True)
    T, E, k, bm = first
    assert _compare(_ids(T, E, k, T + E, bad=(T // 2, 1)), E, bm) == 1
    T, E, k, bm = second
    assert _compare(_ids(T, E, k, T + E + 1), E, bm) == 0


def test_align_noalloc_without_flag_output_and_empty_batch():
    print("align_noalloc flags=None, T=0", flush=True)
    ids_np = _ids(300, 32, 3, 9)
    ids = to_gpu(ids_np)
    ref = ops.align(ids, 32, 32)
    got = ops.align_noalloc(ids, 32, 32)
    torch.cuda.synchronize()
    for key in KEYS:
        assert torch.equal(got[key], ref[key]), key
    empty = torch.empty((0, 4), dtype=torch.int32, device="cuda")
    got = ops.align_noalloc(empty, 8, 16)
    torch.cuda.synchronize()
    assert int(got["num_padded"].item()) == 0
    assert torch.all(got["tile_expert"] == -1)
