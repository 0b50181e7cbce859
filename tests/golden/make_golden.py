"""Writes the stored expected values under tests/golden/ from the oracle only.

The pages print no worked numeric example, so every stored value here comes
from the oracle (``oracle/``), which the CPU tests pin independently.  The
files guard against silent drift of the oracle and give the GPU-side tests
the block lists of the five workloads without recomputing them.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402

# (mesh_rows, mesh_cols, row, col, causal, kv_rotate) of the five workloads.
WORKLOAD_TILES = {
    "1": (2, 2, 0, 0, False, False),
    "2": (4, 4, 2, 2, False, False),
    "3": (4, 4, 2, 2, True, True),
    "4": (8, 8, 4, 4, True, True),
    "5": (16, 4, 8, 2, True, True),
}


def main():
    bl = {k: [list(b) for b in oracle.block_list_ref(*v)] for k, v in WORKLOAD_TILES.items()}
    with open(os.path.join(HERE, "block_lists.json"), "w") as f:
        json.dump({"tiles": WORKLOAD_TILES, "blocks": bl}, f, separators=(",", ":"))

    # A tiny causal tile: 2x2 mesh, rotated, tile (1, 0), L = 3, GQA 2/1, d = 4,
    # inputs quantised to multiples of 1/8 so they are exact in any format.
    r = np.random.default_rng(2024)
    q = np.round(r.standard_normal((6, 2, 4)) * 8) / 8
    k = np.round(r.standard_normal((6, 1, 4)) * 8) / 8
    v = np.round(r.standard_normal((6, 1, 4)) * 8) / 8
    qset, kvset = oracle.mesh_tile_sets_ref(2, 2, 1, 0, True)
    o, lse = oracle.tile_rows_ref(q, k, v, qset, kvset, 3, True, 0.5)
    with open(os.path.join(HERE, "tiny_tile.json"), "w") as f:
        json.dump({"mesh": [2, 2], "tile": [1, 0], "part_len": 3, "causal": True,
                   "kv_rotate": True, "scale": 0.5, "q_parts": qset, "kv_parts": kvset,
                   "q": q.tolist(), "k": k.tolist(), "v": v.tolist(),
                   "o": o.tolist(), "lse": lse.tolist()}, f)

    # The backward of the same tile: dO quantised the same way; the rows' final
    # lse and D over the whole sequence (all four partitions), then the tile's
    # gradient shares.
    do = np.round(r.standard_normal((6, 2, 4)) * 8) / 8
    kall = np.round(r.standard_normal((12, 1, 4)) * 8) / 8
    vall = np.round(r.standard_normal((12, 1, 4)) * 8) / 8
    kall[[p * 3 + i for p in kvset for i in range(3)]] = k
    vall[[p * 3 + i for p in kvset for i in range(3)]] = v
    qpos = oracle.tile_positions_ref(qset, 3)
    o_f, lse_f = oracle.attention_ref(q, kall, vall, qpos, np.arange(12), True, 0.5)
    delta = oracle.bwd_delta_ref(o_f, do)
    dq, dk, dv = oracle.tile_bwd_ref(q, k, v, do, lse_f, delta, qset, kvset, 3, True, 0.5)
    with open(os.path.join(HERE, "tiny_tile_bwd.json"), "w") as f:
        json.dump({"mesh": [2, 2], "tile": [1, 0], "part_len": 3, "causal": True, "scale": 0.5,
                   "q_parts": qset, "kv_parts": kvset, "q": q.tolist(), "k_all": kall.tolist(),
                   "v_all": vall.tolist(), "do": do.tolist(), "lse": lse_f.tolist(),
                   "delta": delta.tolist(), "dq": dq.tolist(), "dk": dk.tolist(),
                   "dv": dv.tolist()}, f)


if __name__ == "__main__":
    main()
