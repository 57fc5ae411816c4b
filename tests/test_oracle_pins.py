"""The CPU oracle against its pins (no GPU needed)."""

import numpy as np
import pytest

import pinlib
from gen import config_inputs, generate, random_case


def test_hand_worked_example():
    pinlib.check_hand_example()


def test_bruteforce_exhaustive_T3_K2_E4():
    assert pinlib.check_bruteforce_exhaustive(T=3, K=2, E=4, Rs=(1, 2, 4)) == 5 ** 6 * 3 * 3


def test_bruteforce_exhaustive_T2_K2_E6():
    assert pinlib.check_bruteforce_exhaustive(T=2, K=2, E=6, Rs=(1, 2, 3, 6)) == 7 ** 4 * 4 * 3


def test_bruteforce_exhaustive_T5_K1_E4():
    pinlib.check_bruteforce_exhaustive(T=5, K=1, E=4, Rs=(1, 2, 4))


def test_bruteforce_dispatch_combine():
    pinlib.check_bruteforce_dispatch_combine(seed=0, cases=300)


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_layout_invariants_full_configs(cfg):
    pinlib.check_layout_invariants(config_inputs(cfg, with_x=False))


@pytest.mark.parametrize("seed", range(4))
def test_layout_invariants_random(seed):
    inp = random_case(seed, 257, 8, 24, 5, 6, 7, mask=0.2, dup=0.3)
    pinlib.check_layout_invariants(inp)


def test_special_cases():
    pinlib.check_special_cases()


@pytest.mark.parametrize("cfg", [0, 3])
def test_dispatch_identity_combine_configs(cfg):
    pinlib.check_identity_combine(config_inputs(cfg))


@pytest.mark.parametrize("cfg", [1, 2, 4])
def test_dispatch_identity_combine_config_routing_small_rows(cfg):
    """The full routing of the large configs with short rows (routing does not
    depend on the row length)."""
    inp = config_inputs(cfg, with_x=False)
    small = generate(inp.T, 64, inp.E, inp.K, inp.R, inp.C, seed=99)
    inp.x = small.x
    inp.H = 64
    pinlib.check_identity_combine(inp)


def test_identity_combine_with_duplicates_and_masks():
    pinlib.check_identity_combine(random_case(5, 300, 40, 16, 6, 4, 3, mask=0.25, dup=0.4))


@pytest.mark.parametrize("seed", range(3))
def test_combine_fp64_bound(seed):
    pinlib.check_combine_fp64(seed)


def test_ll_config3():
    pinlib.check_ll(config_inputs(3))


def test_ll_random_with_masks_dups_and_overflow():
    inp = random_case(3, 40, 16, 8, 4, 2, 1, mask=0.2, dup=0.5, slots=12)
    pinlib.check_ll(inp)


@pytest.mark.parametrize("seed", range(3))
def test_ll_combine_fp64_bound(seed):
    pinlib.check_ll_fp64(seed)


def test_bf16_edges():
    pinlib.check_bf16_edges()


def test_bf16_all_fp32_patterns():
    pinlib.check_bf16_patterns(step=1)


# ------------------------------------------------------------------- NEXT rows


def test_ll_rank_mask_config3():
    inp = config_inputs(3)
    m = np.zeros(inp.R, np.int32)
    m[[3, 17, 31]] = 1
    pinlib.check_ll_rank_mask(inp, m)


def test_ll_rank_mask_random():
    inp = random_case(8, 50, 24, 16, 4, 8, 1, mask=0.1, dup=0.3, slots=60)
    pinlib.check_ll_rank_mask(inp, np.array([0, 1, 0, 0, 1, 1, 0, 0], np.int32))


def test_ll_rank_mask_extremes():
    pinlib.check_ll_mask_extremes(random_case(9, 30, 16, 8, 3, 4, 1, slots=30))


@pytest.mark.parametrize("seed", range(3))
def test_combine_bias(seed):
    pinlib.check_combine_bias(seed)


@pytest.mark.parametrize("seed", range(3))
def test_lb_ops(seed):
    pinlib.check_lb_ops(seed)


def test_e4m3_rounding():
    pinlib.check_e4m3()


def test_ll_fp8_config3_shape():
    inp = config_inputs(3)
    pinlib.check_ll_fp8(inp)


def test_ll_fp8_masked_small():
    inp = random_case(4, 40, 256, 16, 4, 4, 1, mask=0.2, slots=40)
    pinlib.check_ll_fp8(inp, rank_mask=np.array([0, 1, 0, 0], np.int32))


def test_tie_rounding():
    pinlib.check_tie_rounding()


def test_sum_order():
    pinlib.check_sum_order()


def test_fma_and_bias_order():
    pinlib.check_fma_and_bias_order()


def test_ll_fp8_zero_and_tiny_blocks():
    pinlib.check_ll_fp8(pinlib.fp8_edge_case())


def test_ll_fp8_nonfinite_blocks():
    pinlib.check_ll_fp8_nonfinite()


@pytest.mark.parametrize("seed", range(3))
def test_layout_rank_mask_random(seed):
    inp = random_case(20 + seed, 150, 8, 24, 5, 6, 4, mask=0.1, dup=0.2)
    m = np.zeros(6, np.int32)
    m[[seed % 6, (seed + 3) % 6]] = 1
    pinlib.check_layout_rank_mask(inp, m)


def test_layout_rank_mask_full_config():
    inp = config_inputs(2, with_x=False)
    inp.x = random_case(0, inp.T, 8, inp.E, inp.K, inp.R, inp.C).x
    m = np.zeros(inp.R, np.int32)
    m[[0, 7, 31]] = 1
    pinlib.check_layout_rank_mask(inp, m)


def test_layout_rank_mask_exhaustive_tiny():
    """Every table over {-1, 0..3} for T=2, K=2 under every mask of R=2."""
    import itertools
    for flat in itertools.product(range(-1, 4), repeat=4):
        idx = np.array(flat, np.int64).reshape(2, 2)
        for mk in itertools.product((0, 1), repeat=2):
            m = np.array(mk, np.int32)
            for C in (1, 3):
                L = __import__("oracle").layout(idx, 4, 2, C, rank_mask=m)
                B = pinlib.brute_layout(pinlib.masked_topk(idx, 4, 2, m), 4, 2, C)
                pinlib._compare_layout(L, B, 2, 2, C)


@pytest.mark.parametrize("seed", range(3))
def test_combine_rank_mask(seed):
    pinlib.check_combine_rank_mask(seed)


def test_ll_combine_fp8_reduces_to_bf16():
    pinlib.check_ll_combine_fp8(config_inputs(3))


def test_ll_combine_fp8_masked_random():
    inp = random_case(12, 40, 384, 16, 4, 4, 1, mask=0.2, dup=0.2, slots=40)
    pinlib.check_ll_combine_fp8(inp, rank_mask=np.array([0, 0, 1, 0], np.int32), seed=1)
