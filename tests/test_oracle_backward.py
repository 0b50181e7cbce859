"""Pins of the backward oracle (CPU): torch autograd, finite differences,
closed forms, and the sum of the tiles' shares over a whole mesh."""
import pytest

import oracle
from tests import oracle_pins as pins

B = oracle.attention_bwd_ref


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_autograd(causal):
    pins.check_bwd_autograd(B, causal)


def test_matches_autograd_without_gqa():
    pins.check_bwd_autograd(B, True, hq=3, hkv=3, nq=6, nk=10, d=8, seed=30)


def test_finite_differences():
    pins.check_bwd_finite_differences(B)


def test_zero_query_closed_forms():
    pins.check_bwd_zero_query(B)


def test_empty_rows_contribute_nothing():
    pins.check_bwd_empty_rows(B)


@pytest.mark.parametrize("R,C,rot", [(2, 2, True), (3, 2, True), (2, 3, False), (4, 1, True), (1, 3, True)])
def test_tile_shares_sum_to_the_gradient(R, C, rot):
    pins.check_bwd_tile_sum(oracle.tile_bwd_ref, oracle.mesh_tile_sets_ref, R, C, rot=rot)


def test_delta_is_rowwise_dot():
    import numpy as np
    r = np.random.default_rng(0)
    o, do = r.standard_normal((5, 3, 4)), r.standard_normal((5, 3, 4))
    d = oracle.bwd_delta_ref(o, do)
    for i in range(5):
        for h in range(3):
            assert abs(d[i, h] - sum(float(o[i, h, t]) * float(do[i, h, t]) for t in range(4))) < 1e-13
