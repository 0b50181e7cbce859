"""A tile computed in the order of the library's greedy plan: each step's
blocks through the tile forward, folded into a running (O, lse) by the merge,
equal to the oracle over the whole tile; and at the step where the plan sends
a Q slot's partial back, that slot's running rows already equal the oracle
over all of the slot's blocks (the plan only sends finished rows)."""
import math

import numpy as np
import pytest

import oracle
import workloads
from tests.conftest import gpu_available
from tests.parity import compare, run_tile, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a HIP GPU")]

COSTS = {
    "balanced": dict(recv_q_s=1.0, recv_kv_s=1.0, send_o_s=1.0, full_block_s=1.0, diag_block_s=0.5),
    "compute-bound": dict(recv_q_s=0.25, recv_kv_s=0.5, send_o_s=0.25, full_block_s=1.0,
                          diag_block_s=0.5),
    "comm-bound": dict(recv_q_s=4.0, recv_kv_s=2.0, send_o_s=4.0, full_block_s=1.0, diag_block_s=0.5),
}

CASES = [
    # L, mesh, tile, causal, rotate, Hq, Hkv
    (48, (3, 3), (1, 1), True, True, 4, 2),
    (40, (4, 4), (2, 2), True, True, 8, 2),
    (33, (2, 3), (1, 2), False, True, 4, 4),
    (64, (8, 2), (4, 1), True, True, 4, 1),
    (24, (4, 2), (2, 0), True, False, 4, 2),
]


@pytest.mark.parametrize("regime", sorted(COSTS))
@pytest.mark.parametrize("case", CASES, ids=[f"L{c[0]}-{c[1][0]}x{c[1][1]}-t{c[2]}-c{int(c[3])}"
                                             f"-r{int(c[4])}" for c in CASES])
def test_tile_in_planned_order(case, regime):
    import torch
    import long_context_distributed_amd as mat
    L, (R, C), (r, c), causal, rot, hq, hkv = case
    w = workloads.small("bf16", L, R, C, r, c, causal, rot, hq, hkv, 128)
    say(f"[case] planned order {w.name} costs {regime}")
    steps = mat.plan(R, C, r, c, causal, rot, COSTS[regime])
    t = run_tile(w)
    scale = 1.0 / math.sqrt(128)
    ref_o, ref_lse = oracle.tile_rows_ref(t["q"], t["k"], t["v"], t["q_parts"], t["kv_parts"], L,
                                          causal, scale)
    rows = t["q"].shape[0] * hq
    o_run = torch.zeros_like(t["o"])
    lse_run = torch.full_like(t["lse"], -math.inf)
    n_blocks = 0
    for st in steps:
        if st["comm"] == mat.COMM_SEND_O:
            # the partial of this Q slot leaves now: its rows must be final
            s = st["slot"]
            sl = slice(s * L, (s + 1) * L)
            compare(o_run[sl], lse_run[sl], ref_o[sl], ref_lse[sl], "bf16",
                    what=f"Q slot {s} at its send step")
        if not st["blocks"]:
            continue
        n_blocks += len(st["blocks"])
        o_j, lse_j = mat.tile_fwd(t["q"], t["k"], t["v"], st["blocks"], L, scale)
        o_m, lse_m = mat.lse_merge(torch.stack([o_run.view(rows, 128), o_j.view(rows, 128)]),
                                   torch.stack([lse_run.view(rows), lse_j.view(rows)]))
        o_run, lse_run = o_m.view_as(o_j), lse_m.view_as(lse_j)
    assert n_blocks == sum(1 for b in t["blocks"] if b[4] != 2)
    compare(o_run, lse_run, ref_o, ref_lse, "bf16", what=f"whole tile in planned order ({len(steps)} steps)")
    assert np.isfinite(steps[-1]["end_s"])
