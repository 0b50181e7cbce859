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


def test_tiny_tile_backward_matches_oracle():
    with open(os.path.join(HERE, "tiny_tile_bwd.json")) as f:
        g = json.load(f)
    q, kall, vall, do = (np.array(g[x]) for x in ("q", "k_all", "v_all", "do"))
    L = g["part_len"]
    kv_rows = [p * L + i for p in g["kv_parts"] for i in range(L)]
    qpos = oracle.tile_positions_ref(g["q_parts"], L)
    o_f, lse_f = oracle.attention_ref(q, kall, vall, qpos, np.arange(kall.shape[0]), g["causal"],
                                      g["scale"])
    delta = oracle.bwd_delta_ref(o_f, do)
    assert np.allclose(lse_f, np.array(g["lse"]), rtol=0, atol=1e-14)
    assert np.allclose(delta, np.array(g["delta"]), rtol=0, atol=1e-14)
    dq, dk, dv = oracle.tile_bwd_ref(q, kall[kv_rows], vall[kv_rows], do, lse_f, delta,
                                     g["q_parts"], g["kv_parts"], L, g["causal"], g["scale"])
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert np.allclose(got, np.array(g[name]), rtol=0, atol=1e-13), name
