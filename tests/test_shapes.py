"""Host logic of the workload shapes: the token-bucket view of a shape and
the default tile height, against the block_m choices that a tile sweep on
one MI355X measured within 2% of the fastest (bench.py --tile-sweep; each
of them passed its bit-exact accuracy gate)."""
import pytest

from quantized_mixture_experts_moe_amd.shapes import (A8W4_LARGE, A8W4_TP2, A8W4_TP4,
                                                      default_block_m, shape_by_name)

# (share, tokens) -> the block_m values within 2% of the fastest step.
MEASURED_GOOD = {
    ("a8w4_large", 1): {16, 32, 64}, ("a8w4_large", 16): {16, 32, 64},
    ("a8w4_large", 64): {16, 32, 64}, ("a8w4_large", 256): {16, 32},
    ("a8w4_large", 1024): {64, 128}, ("a8w4_large", 4096): {128},
    ("a8w4_large", 8192): {128},
    ("a8w4_tp2", 1): {16, 32}, ("a8w4_tp2", 16): {16, 32, 64}, ("a8w4_tp2", 64): {16, 32},
    ("a8w4_tp2", 256): {16, 32}, ("a8w4_tp2", 1024): {32, 64, 128},
    ("a8w4_tp2", 4096): {128}, ("a8w4_tp2", 8192): {64},
    ("a8w4_tp4", 1): {16, 32}, ("a8w4_tp4", 16): {16, 32}, ("a8w4_tp4", 64): {16, 32},
    ("a8w4_tp4", 256): {16, 32}, ("a8w4_tp4", 1024): {64}, ("a8w4_tp4", 4096): {128},
    ("a8w4_tp4", 8192): {64},
}


@pytest.mark.parametrize("share,T", sorted(MEASURED_GOOD))
def test_default_block_m_is_a_measured_good_choice(share, T):
    assert default_block_m(shape_by_name(f"{share}@T{T}")) in MEASURED_GOOD[(share, T)]


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
