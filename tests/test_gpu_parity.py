"""GPU parity of the tile forward and the LSE merge against the oracle, on
oracle-sized tiles that span several LDS tiles and ragged tails.

Every call goes through the C ABI (ctypes binding) into the HIP kernels.
"""
import math

import numpy as np
import pytest

import oracle
import workloads
from tests.conftest import gpu_available
from tests.parity import compare, expected_empty_rows, run_tile, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a HIP GPU")]

SMALL = [
    # dtype, L, mesh, tile, causal, rotate, Hq, Hkv, d
    ("bf16", 64, (2, 2), (0, 0), True, True, 4, 2, 128),
    ("bf16", 17, (2, 2), (0, 1), True, True, 4, 1, 128),     # ragged; empty rows
    ("bf16", 129, (4, 4), (2, 2), True, True, 8, 1, 128),    # G=8, ragged, 3 kinds
    ("bf16", 128, (4, 4), (1, 3), True, True, 2, 2, 128),    # MHA
    ("bf16", 1, (2, 3), (1, 1), True, True, 4, 4, 128),      # one-token partitions
    ("bf16", 16, (1, 1), (0, 0), True, False, 4, 2, 128),    # diagonal block only
    ("bf16", 96, (3, 2), (1, 0), False, False, 6, 2, 128),   # non-causal, G=3
    ("bf16", 200, (2, 4), (1, 2), True, True, 16, 2, 128),   # G=8 with 2 head groups
    ("bf16", 100, (2, 2), (1, 0), True, True, 12, 1, 128),   # G=12: all 12 waves on heads of one group
    ("bf16", 70, (2, 3), (0, 2), True, True, 10, 2, 128),    # G=5: one head per workgroup, 5 head groups
    ("bf16", 90, (4, 2), (2, 1), True, False, 4, 2, 128),    # causal with contiguous KV order
    ("f32", 64, (2, 2), (0, 0), False, False, 1, 1, 64),
    ("f32", 33, (2, 2), (1, 1), True, True, 2, 1, 64),
    ("f32", 40, (4, 2), (2, 1), True, True, 4, 2, 128),
    ("f32", 150, (4, 4), (2, 1), True, True, 6, 2, 128),   # several key tiles per wave, ragged, G=3
    ("f32", 200, (3, 2), (1, 0), True, False, 2, 2, 64),   # contiguous KV, two diagonal blocks
    ("f32", 7, (2, 2), (1, 1), True, True, 3, 1, 64),      # fewer keys than waves
    ("f32", 300, (2, 2), (1, 0), True, True, 2, 1, 64),    # causal, several 64-row blocks per diagonal
    ("f32", 1000, (2, 2), (1, 0), False, True, 2, 1, 64),  # long non-causal rows
]


def _wl(case, seed=0):
    dtype, L, (R, C), (r, c), causal, rot, hq, hkv, d = case
    return workloads.small(dtype, L, R, C, r, c, causal, rot, hq, hkv, d, seed=seed)


@pytest.mark.parametrize("case", SMALL, ids=[f"{c[0]}-L{c[1]}-{c[2][0]}x{c[2][1]}-t{c[3]}"
                                             f"-c{int(c[4])}-G{c[6]}/{c[7]}-d{c[8]}" for c in SMALL])
def test_tile_matches_oracle_all_rows(case):
    w = _wl(case)
    say(f"[case] {w.name}")
    t = run_tile(w)
    ref_o, ref_lse = oracle.tile_rows_ref(t["q"], t["k"], t["v"], t["q_parts"], t["kv_parts"],
                                          w.part_len, w.causal, 1.0 / math.sqrt(w.head_dim))
    compare(t["o"], t["lse"], ref_o, ref_lse, w.dtype, what=w.name)
    empty = expected_empty_rows(t["q_parts"], t["kv_parts"], w.part_len, w.causal)
    assert np.array_equal(np.isneginf(t["lse"].cpu().numpy()).all(axis=1), empty)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_zero_query_closed_form_on_gpu(dtype, d):
    """Q = 0: lse = ln(visible count) and O = mean of visible V, with the count
    n_before*L + (u+1 if the own partition is held) - pins the mask on the GPU."""
    import torch
    w = workloads.small(dtype, 96, 4, 4, 2, 2, True, True, 4, 2, d)
    t = run_tile(w)
    q0 = torch.zeros_like(t["q"])
    t0 = run_tile(w, inputs=(q0, t["k"], t["v"]))
    lse = t0["lse"].cpu().numpy().astype(np.float64)
    o = t0["o"].float().cpu().numpy().astype(np.float64)
    v = t["v"].float().cpu().numpy().astype(np.float64)
    L = w.part_len
    kpos = oracle.tile_positions_ref(t["kv_parts"], L)
    g = w.heads_q // w.heads_kv
    worst_o = 0.0
    for s, qp in enumerate(t["q_parts"]):
        n_before = sum(1 for kp in t["kv_parts"] if kp < qp)
        own = qp in t["kv_parts"]
        for u in range(L):
            cnt = n_before * L + (u + 1 if own else 0)
            i = s * L + u
            if cnt == 0:
                assert np.all(np.isneginf(lse[i])) and np.all(o[i] == 0)
                continue
            assert np.max(np.abs(lse[i] - math.log(cnt))) < 1e-5, (s, u, lse[i], cnt)
            vis = kpos <= qp * L + u
            for h in range(w.heads_q):
                mean = v[vis, h // g, :].mean(axis=0)
                worst_o = max(worst_o, float(np.max(np.abs(o[i, h] - mean))))
    say(f"[closed-form] {dtype}: max|dO|={worst_o:.3e}")
    assert worst_o <= (2e-2 if dtype == "bf16" else 1e-5)


def test_deterministic_and_canaries():
    """Two runs are bitwise identical; guard bands around the outputs stay untouched."""
    import torch
    import long_context_distributed_amd as mat
    w = workloads.small("bf16", 130, 4, 4, 2, 2, True, True, 8, 2, 128)
    t = run_tile(w)
    n_o, n_l = t["o"].numel(), t["lse"].numel()
    pad = 4096
    big_o = torch.full((n_o + 2 * pad,), -7.0, dtype=torch.bfloat16, device="cuda")
    big_l = torch.full((n_l + 2 * pad,), 3.5, dtype=torch.float32, device="cuda")
    o2 = big_o[pad:pad + n_o].view(t["o"].shape)
    l2 = big_l[pad:pad + n_l].view(t["lse"].shape)
    mat.tile_fwd(t["q"], t["k"], t["v"], t["blocks"], w.part_len, 1.0 / math.sqrt(128),
                 out=o2, lse=l2)
    torch.cuda.synchronize()
    assert torch.equal(o2, t["o"]) and torch.equal(l2, t["lse"]), "not deterministic"
    assert torch.all(big_o[:pad] == -7.0) and torch.all(big_o[-pad:] == -7.0), "O canary hit"
    assert torch.all(big_l[:pad] == 3.5) and torch.all(big_l[-pad:] == 3.5), "lse canary hit"


@pytest.mark.parametrize("dtype,d,n", [("bf16", 128, 5), ("f32", 64, 5), ("bf16", 64, 5),
                                       ("f32", 128, 5), ("bf16", 128, 1), ("bf16", 128, 2),
                                       ("bf16", 128, 16), ("bf16", 128, 20), ("f32", 64, 33),
                                       ("bf16", 24, 3), ("f32", 12, 7), ("bf16", 128, 64),
                                       ("f32", 128, 64)])
def test_merge_matches_oracle(dtype, d, n):
    import torch
    import long_context_distributed_amd as mat
    r = np.random.default_rng(5)
    rows = 3001
    o = r.standard_normal((n, rows, d))
    lse = 4.0 * r.standard_normal((n, rows))
    lse[min(1, n - 1), ::3] = -np.inf  # dead partial rows
    lse[:, 7] = -np.inf            # an all-dead row
    lse[:, 9] = 80.0               # large equal values
    o[np.isneginf(lse)] = np.nan   # rows of dead partials must not be read
    tdt = workloads.torch_dtype(dtype)
    o_t = torch.from_numpy(o).to(tdt).cuda()
    l_t = torch.from_numpy(lse).float().cuda()
    mo, ml = mat.lse_merge(o_t, l_t)
    ro, rl = oracle.lse_merge_ref(o_t.cpu(), l_t.cpu())
    tol_o, tol_l = (2e-2, 1e-3) if dtype == "bf16" else (1e-5, 1e-5)
    got_o = mo.float().cpu().numpy()
    got_l = ml.cpu().numpy().astype(np.float64)
    assert not np.any(np.isnan(got_o))
    assert np.array_equal(np.isneginf(got_l), np.isneginf(rl))
    fin = np.isfinite(rl)
    say(f"[merge] {dtype} d={d}: max|dO|={np.max(np.abs(got_o - ro)):.3e} "
        f"max|dlse|={np.max(np.abs(got_l[fin] - rl[fin])):.3e}")
    assert np.max(np.abs(got_o - ro)) <= tol_o
    assert np.max(np.abs(got_l[fin] - rl[fin])) <= tol_l
    # lse output is optional
    mo2, none = mat.lse_merge(o_t, l_t, want_lse=False)
    assert none is None and torch.equal(mo2, mo)


@pytest.mark.parametrize("dtype,causal", [("bf16", True), ("bf16", False), ("f32", True)])
def test_mesh_row_siblings_merge_to_full_attention(dtype, causal):
    """Tiles (r, 0..C-1) of one mesh row, merged on the GPU, equal the oracle's
    attention of that row's Q over the union of their KV sets."""
    import torch
    import long_context_distributed_amd as mat
    d = 128 if dtype == "bf16" else 64
    w = workloads.small(dtype, 80, 4, 3, 2, 0, causal, True, 4, 2, d)
    outs = [run_tile(w, col=c) for c in range(w.mesh_cols)]
    rows = outs[0]["q"].shape[0] * w.heads_q
    o_parts = torch.stack([t["o"].reshape(rows, d) for t in outs])
    l_parts = torch.stack([t["lse"].reshape(rows) for t in outs])
    mo, ml = mat.lse_merge(o_parts, l_parts)
    kv_all = sum((t["kv_parts"] for t in outs), [])
    k_all = torch.cat([t["k"] for t in outs])
    v_all = torch.cat([t["v"] for t in outs])
    ref_o, ref_lse = oracle.tile_rows_ref(outs[0]["q"], k_all, v_all, outs[0]["q_parts"], kv_all,
                                          w.part_len, causal, 1.0 / math.sqrt(d))
    compare(mo.view_as(outs[0]["o"]), ml.view_as(outs[0]["lse"]), ref_o, ref_lse, dtype,
            what=f"mesh-row merge {dtype} causal={causal}")


def test_per_kv_slot_subtiles_merge_to_single_launch():
    """The same kernel on each one-KV-slot subset of a tile's blocks, merged,
    equals the single launch over all blocks."""
    import torch
    import long_context_distributed_amd as mat
    w = workloads.small("bf16", 72, 6, 2, 3, 1, True, True, 8, 2, 128)
    t = run_tile(w)
    parts = []
    for j in range(w.mesh_rows):
        sub = [b for b in t["blocks"] if b[1] == j]
        parts.append(run_tile(w, blocks=sub, inputs=(t["q"], t["k"], t["v"])))
    rows = t["q"].shape[0] * w.heads_q
    mo, ml = mat.lse_merge(torch.stack([p["o"].reshape(rows, 128) for p in parts]),
                           torch.stack([p["lse"].reshape(rows) for p in parts]))
    got_o = mo.float().cpu().numpy()
    want_o = t["o"].float().cpu().numpy().reshape(rows, 128)
    got_l = ml.cpu().numpy()
    want_l = t["lse"].cpu().numpy().reshape(rows)
    assert np.array_equal(np.isneginf(got_l), np.isneginf(want_l))
    fin = np.isfinite(want_l)
    assert np.max(np.abs(got_o - want_o)) <= 2e-2
    assert np.max(np.abs(got_l[fin] - want_l[fin])) <= 1e-3


@pytest.mark.parametrize("R,C,r,c,L,hq,hkv", [(8, 2, 4, 1, 48, 4, 2), (16, 2, 8, 1, 40, 4, 2),
                                             (16, 1, 5, 0, 33, 8, 1)])
def test_running_pairwise_merge_one_kv_slot_at_a_time(R, C, r, c, L, hq, hkv):
    """A tile computed one KV slot at a time, in rotation order, each partial
    folded into a running result by a two-way merge whose bf16 output is the
    next step's input (n-1 bf16 roundings of O), equals the oracle over the
    whole tile within the bf16 bounds.  8 and 16 KV slots."""
    import torch
    import long_context_distributed_amd as mat
    w = workloads.small("bf16", L, R, C, r, c, True, True, hq, hkv, 128)
    say(f"[case] running merge {w.name}")
    t = run_tile(w)
    rows = t["q"].shape[0] * hq
    o_run = lse_run = None
    for j in range(R):
        step_blocks = [b for b in t["blocks"] if b[1] == j]
        o_j, lse_j = mat.tile_fwd(t["q"], t["k"], t["v"], step_blocks, L)
        if o_run is None:
            o_run, lse_run = o_j, lse_j
            continue
        o_m, lse_m = mat.lse_merge(torch.stack([o_run.view(rows, 128), o_j.view(rows, 128)]),
                                   torch.stack([lse_run.view(rows), lse_j.view(rows)]))
        o_run, lse_run = o_m.view_as(o_j), lse_m.view_as(lse_j)
    ref_o, ref_lse = oracle.tile_rows_ref(t["q"], t["k"], t["v"], t["q_parts"], t["kv_parts"],
                                          L, True, 1.0 / math.sqrt(128))
    compare(o_run, lse_run, ref_o, ref_lse, "bf16", what=f"running merge over {R} KV slots")


@pytest.mark.parametrize("L,mesh,tile,hq,hkv,d", [(4096, (2, 2), (1, 0), 4, 2, 64),
                                                  (2048, (4, 2), (2, 1), 8, 2, 128)])
def test_f32_long_causal_partitions_sampled_rows(L, mesh, tile, hq, hkv, d):
    """Float32 causal tiles with long partitions (thousands of keys per
    diagonal block), checked on seeded sampled rows plus the edge rows of
    every Q slot at the float32 bound."""
    w = workloads.small("f32", L, mesh[0], mesh[1], tile[0], tile[1], True, True, hq, hkv, d)
    say(f"[case] {w.name}")
    t = run_tile(w)
    rows = workloads.sample_rows(t["q"].shape[0], hq, hkv, L, n_sample=512, seed=4)
    ref_o, ref_lse = oracle.tile_rows_ref(t["q"], t["k"], t["v"], t["q_parts"], t["kv_parts"], L, True,
                                          1.0 / math.sqrt(d), rows=rows)
    compare(t["o"], t["lse"], ref_o, ref_lse, "f32", rows=rows, what=w.name)
