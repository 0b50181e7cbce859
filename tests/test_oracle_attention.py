"""Pins of the attention oracle (CPU only)."""
import pytest

import oracle
from tests import oracle_pins as pins


def attention(q, k, v, qp, kp, causal, scale):
    return oracle.attention_ref(q, k, v, qp, kp, causal, scale)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("hq,hkv", [(1, 1), (4, 2), (8, 1)])
def test_matches_torch_sdpa_and_scipy_logsumexp(causal, hq, hkv):
    pins.check_sdpa(attention, causal, hq=hq, hkv=hkv)


def test_zero_query_gives_mean_and_log_count():
    pins.check_zero_query(attention)
    pins.check_zero_query(attention, L=3, q_parts=(0, 1, 2), kv_parts=(1, 3), hq=4, hkv=2)


def test_single_visible_key():
    pins.check_single_key(attention)


@pytest.mark.parametrize("causal", [False, True])
def test_affine_in_values_and_rows_sum_to_one(causal):
    pins.check_affine_values(attention, causal)


def test_gqa_head_mapping():
    pins.check_gqa_mapping(attention)


@pytest.mark.parametrize("causal", [False, True])
def test_pure_python_brute_force(causal):
    pins.check_brute_force(attention, causal)


def test_large_scores_stay_finite():
    pins.check_large_scores(attention)


def test_key_order_irrelevant_without_mask():
    pins.check_key_permutation(attention)


def test_scale_multiplies_scores():
    pins.check_scale_on_scores(attention)


def test_tile_rows_subset_equals_full():
    """Row sampling returns exactly the rows of the full evaluation."""
    import numpy as np
    r = np.random.default_rng(0)
    q = r.standard_normal((8, 4, 8))
    k = r.standard_normal((12, 2, 8))
    v = r.standard_normal((12, 2, 8))
    o, lse = oracle.tile_rows_ref(q, k, v, [3, 1], [1, 0, 3], 4, True, 0.3)
    rows = np.array([[0, 0], [5, 3], [7, 1], [2, 2]])
    so, sl = oracle.tile_rows_ref(q, k, v, [3, 1], [1, 0, 3], 4, True, 0.3, rows=rows)
    assert np.array_equal(so, o[rows[:, 0], rows[:, 1]])
    assert np.array_equal(sl, lse[rows[:, 0], rows[:, 1]])


def test_tile_positions():
    import numpy as np
    assert oracle.tile_positions_ref([2, 0], 3).tolist() == [6, 7, 8, 0, 1, 2]
    assert oracle.tile_positions_ref([], 3).shape == (0,)
