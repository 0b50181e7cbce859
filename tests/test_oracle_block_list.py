"""Pins of the block-list oracle (CPU only)."""
import pytest

import oracle
from tests import oracle_pins as pins


def block_list(R, C, r, c, causal, rot):
    return oracle.block_list_ref(R, C, r, c, causal, rot)


@pytest.mark.parametrize("R,C", [(1, 1), (2, 2), (4, 4), (8, 8), (16, 4), (3, 5), (1, 6), (6, 1)])
def test_geometry(R, C):
    pins.check_block_list_geometry(block_list, R, C)


@pytest.mark.parametrize("R,C", [(1, 1), (2, 2), (4, 4), (8, 8), (16, 4), (3, 5), (1, 6), (6, 1)])
def test_kinds(R, C):
    pins.check_block_list_kinds(block_list, R, C)


@pytest.mark.parametrize("R,C", [(1, 1), (2, 2), (4, 4), (8, 8), (16, 4), (3, 5), (1, 6), (6, 1)])
def test_contiguous_tiling(R, C):
    pins.check_block_list_contiguous(block_list, R, C)


def test_fp32_workload_tile_literal():
    pins.check_block_list_fp32_workload_tile(block_list)


@pytest.mark.parametrize("L", [2, 3, 5])
def test_classification_independent_of_length(L):
    for r in range(4):
        for c in range(4):
            assert oracle.block_list_ref(4, 4, r, c, True, True, part_len=L) == \
                oracle.block_list_ref(4, 4, r, c, True, True)


def test_one_token_partitions_have_no_diagonal():
    kinds = [b[4] for b in oracle.block_list_ref(2, 2, 0, 0, True, True, part_len=1)]
    assert oracle.DIAG not in kinds


def test_rejects_bad_geometry():
    with pytest.raises(ValueError):
        oracle.block_list_ref(0, 2, 0, 0, True, True)
    with pytest.raises(ValueError):
        oracle.block_list_ref(2, 2, 2, 0, True, True)
