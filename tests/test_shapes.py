"""Host logic of the workload shapes and the gfx950 tile table: the token-
bucket view of a shape, and the default tile height (the library's table,
else its rule) against the block_m choices that the gated tile sweep on one
MI355X measured within 2% of the fastest (bench.py --tile-sweep; each passed
its bit-exact accuracy gate; profiles/tile_table_sweep.md)."""
import os
import re

import pytest

from quantized_mixture_experts_moe_amd.shapes import (A8W4_LARGE, A8W4_TP2, A8W4_TP4,
                                                      SCHEME_CODE, default_block_m,
                                                      shape_by_name)

TABLE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                     "quantized_mixture_experts_moe_amd", "csrc", "tile_table.inc")

# (workload, tokens) -> the block_m values within 2% of the fastest step.
MEASURED_GOOD = {
    ("a8w4_large", 1): {16, 32}, ("a8w4_large", 16): {16, 32, 64},
    ("a8w4_large", 64): {16, 32, 64, 128}, ("a8w4_large", 256): {16, 32, 64, 128},
    ("a8w4_large", 1024): {128}, ("a8w4_large", 4096): {128}, ("a8w4_large", 8192): {128},
    ("a8w4_tp2", 1): {16, 32}, ("a8w4_tp2", 16): {16, 32}, ("a8w4_tp2", 64): {16, 32, 64, 128},
    ("a8w4_tp2", 256): {16, 32, 64, 128}, ("a8w4_tp2", 1024): {128}, ("a8w4_tp2", 4096): {128},
    ("a8w4_tp2", 8192): {64},
    ("a8w4_tp4", 1): {16, 32}, ("a8w4_tp4", 16): {16, 32}, ("a8w4_tp4", 64): {16, 32, 64},
    ("a8w4_tp4", 256): {16, 32}, ("a8w4_tp4", 1024): {64, 128}, ("a8w4_tp4", 4096): {128},
    ("a8w4_tp4", 8192): {64},
    ("w4a16_qwen3moe_t128", 128): {32}, ("w8a8_t2048", 2048): {64},
    ("w4a8_qwen3moe_t128", 128): {16, 32, 64}, ("w4a8_qwen3moe_t128", 2048): {64},
    ("w4a16_skewed_t8192", 8192): {128}, ("w4a8_skewed_t8192", 8192): {64, 128},
}


@pytest.mark.parametrize("name,T", sorted(MEASURED_GOOD))
def test_default_block_m_is_a_measured_good_choice(name, T):
    sh = shape_by_name(name).with_tokens(T)
    assert default_block_m(sh) in MEASURED_GOOD[(name, T)]


def _table_rows():
    rows = []
    for line in open(TABLE):
        line = line.strip()
        if not line or line.startswith("//"):
            continue
        nums = [int(v) for v in re.findall(r"-?\d+", line)]
        assert len(nums) == 13, line
        rows.append(nums)
    return rows


def test_tile_table_rows_are_well_formed():
    """Every row: a known scheme, block_m of the four heights, knobs in their
    ranges, and the rows of one shape in strictly ascending token buckets."""
    rows = _table_rows()
    assert rows
    last = {}
    for sc, H, I, E, k, t_max, bm, s1w, s1r, s1runs, s2w, s2p, s2h in rows:
        assert sc in SCHEME_CODE.values() and 1 <= k <= E and t_max >= 1
        assert bm in (16, 32, 64, 128)
        assert s1w in (0, 4, 8) and (s1w != 8 or bm >= 64)
        assert s1r in (0, 4) and s1runs in (-1, 0, 1, 2) and s2h in (-1, 0, 1)
        resident = sc in (1, 2) and I <= 1024
        assert s2w == 0 or (not resident and s2w in (4, 8))
        assert s2p == 0 or (resident and (H // 256) % s2p == 0)
        key = (sc, H, I, E, k)
        assert t_max > last.get(key, 0)
        last[key] = t_max


def test_default_block_m_follows_the_table():
    """Each bucket's row gives the block_m for every token count from the
    previous bucket (exclusive) to its own."""
    prev = {}
    for sc, H, I, E, k, t_max, bm, *_ in _table_rows():
        lib_scheme = {v: n for n, v in SCHEME_CODE.items()}[sc]
        lo = prev.get((sc, H, I, E, k), 0) + 1
        for T in sorted({lo, (lo + t_max) // 2, t_max}):
            from quantized_mixture_experts_moe_amd.shapes import MoEShape
            sh = MoEShape("t", lib_scheme, tokens=T, hidden=H, inter=I, experts=E, topk=k,
                          seed=0)
            assert default_block_m(sh) == bm, (sc, H, I, E, k, T)
        prev[(sc, H, I, E, k)] = t_max


def test_tensor_parallel_shares_split_the_intermediate():
    for share, ways in ((A8W4_TP2, 2), (A8W4_TP4, 4)):
        assert share.inter * ways == A8W4_LARGE.inter
        assert (share.hidden, share.experts, share.topk) == (
            A8W4_LARGE.hidden, A8W4_LARGE.experts, A8W4_LARGE.topk)
        # one GPU's share does 1/ways of the block's useful flops
        assert share.useful_flops() * ways == A8W4_LARGE.useful_flops()


def test_token_buckets_take_leading_rows():
    s = shape_by_name("a8w4_tp4@T16")
    assert (s.tokens, s.tokens_drawn, s.seed) == (16, 8192, A8W4_TP4.seed)
    with pytest.raises(AssertionError):
        shape_by_name("a8w4_tp4@T16384")
