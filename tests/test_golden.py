"""The stored expected values still match the oracle (drift guard, CPU only)."""
import json
import os

import numpy as np

import oracle

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_block_lists_match_oracle():
    with open(os.path.join(HERE, "block_lists.json")) as f:
        g = json.load(f)
    for key, tile in g["tiles"].items():
        assert [list(b) for b in oracle.block_list_ref(*tile)] == g["blocks"][key]
    # the 1M-token workload's tile (4,4) of the 8x8 mesh: KV column 4, own partition first
    kv = [b[3] for b in g["blocks"]["4"] if b[0] == 0]
    assert kv == [36, 44, 52, 60, 4, 12, 20, 28]
    kinds = [b[4] for b in g["blocks"]["4"]]
    assert (kinds.count(0), kinds.count(1), kinds.count(2)) == (35, 1, 28)


def test_tiny_tile_matches_oracle():
    with open(os.path.join(HERE, "tiny_tile.json")) as f:
        g = json.load(f)
    o, lse = oracle.tile_rows_ref(np.array(g["q"]), np.array(g["k"]), np.array(g["v"]),
                                  g["q_parts"], g["kv_parts"], g["part_len"], g["causal"],
                                  g["scale"])
    assert np.allclose(o, np.array(g["o"]), rtol=0, atol=1e-14)
    assert np.allclose(lse, np.array(g["lse"]), rtol=0, atol=1e-14)
