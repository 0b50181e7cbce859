"""Helpers for the GPU parity tests: run a workload's tile through the C-ABI
binding and compare with the oracle on the same seeded inputs.

The library side takes its tile geometry from the library's block list; the
oracle side from the oracle's own block list (the two are also compared
bit-exactly).  Inputs come from ``workloads`` (random numbers only) and the
oracle reads the device values back, so the two sides share no arithmetic.
"""
import math
import sys

import numpy as np

import oracle
import workloads

# Tolerances (max abs error) by dtype: (O, lse).
TOL = {"bf16": (2e-2, 1e-3), "f32": (1e-5, 1e-5)}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def tile_geometry(w, lib_blocks):
    """(q_parts, kv_parts) in slot order from a block list."""
    qp = {b[0]: b[2] for b in lib_blocks}
    kp = {b[1]: b[3] for b in lib_blocks}
    return [qp[i] for i in range(len(qp))], [kp[i] for i in range(len(kp))]


def run_tile(w, row=None, col=None, device="cuda", blocks=None, inputs=None):
    """Forward of tile (row, col) of workload w through the library.

    Returns dict with q, k, v (device), o, lse (device), blocks, q_parts, kv_parts.
    """
    import long_context_distributed_amd as mat
    row = w.tile_row if row is None else row
    col = w.tile_col if col is None else col
    lib_blocks = mat.block_list(w.mesh_rows, w.mesh_cols, row, col, w.causal, w.kv_rotate)
    ref_blocks = oracle.block_list_ref(w.mesh_rows, w.mesh_cols, row, col, w.causal, w.kv_rotate)
    assert lib_blocks == ref_blocks, "library block list differs from the oracle's"
    q_parts, kv_parts = tile_geometry(w, lib_blocks)
    if inputs is None:
        q = workloads.gather(w, "q", q_parts, device)
        k = workloads.gather(w, "k", kv_parts, device)
        v = workloads.gather(w, "v", kv_parts, device)
    else:
        q, k, v = inputs
    use = lib_blocks if blocks is None else blocks
    o, lse = mat.tile_fwd(q, k, v, use, w.part_len, 1.0 / math.sqrt(w.head_dim))
    return dict(q=q, k=k, v=v, o=o, lse=lse, blocks=lib_blocks, q_parts=q_parts,
                kv_parts=kv_parts)


def expected_empty_rows(q_parts, kv_parts, part_len, causal):
    """Boolean [n_q_slots*L] - rows with no visible key.  Closed form: a row of
    partition qp sees a key only if some KV partition kp <= qp is held."""
    out = np.zeros(len(q_parts) * part_len, dtype=bool)
    if not causal:
        return out
    for s, qp in enumerate(q_parts):
        if not any(kp <= qp for kp in kv_parts):
            out[s * part_len:(s + 1) * part_len] = True
    return out


def compare(o_dev, lse_dev, ref_o, ref_lse, dtype, rows=None, what="", tol=None):
    """Max-abs comparison; rows selects (token, head) pairs of o_dev/lse_dev;
    tol = (O, lse) overrides the per-dtype tolerances."""
    to, tl = TOL[dtype] if tol is None else tol
    o = o_dev.float().cpu().numpy().astype(np.float64)
    lse = lse_dev.cpu().numpy().astype(np.float64)
    if rows is not None:
        o = o[rows[:, 0], rows[:, 1]]
        lse = lse[rows[:, 0], rows[:, 1]]
    assert o.shape == ref_o.shape and lse.shape == ref_lse.shape, (o.shape, ref_o.shape)
    ref_inf = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), ref_inf), f"{what}: -inf rows differ"
    assert not np.any(np.isnan(o)), f"{what}: NaN in output"
    err_o = float(np.max(np.abs(o - ref_o))) if o.size else 0.0
    fin = ~ref_inf
    err_l = float(np.max(np.abs(lse[fin] - ref_lse[fin]))) if fin.any() else 0.0
    assert np.all(o[ref_inf] == 0), f"{what}: empty rows must be 0"
    say(f"[parity] {what}: max|dO|={err_o:.3e} (tol {to}) max|dlse|={err_l:.3e} (tol {tl})")
    assert err_o <= to, f"{what}: O error {err_o} > {to}"
    assert err_l <= tl, f"{what}: lse error {err_l} > {tl}"
    return err_o, err_l
